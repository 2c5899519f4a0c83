/*
 * moe.h -- C ABI of an MI355X (gfx950) Mixture-of-Experts FFN layer forward.
 *
 * The layer (intelliparadigm.com, "MoE模型高效推理：CANN算子库优化实践", section 2.1,
 * the moe_layer pseudo-code; gitcode.csdn.net, "ops-transformer 仓库 - MoE 算子优化实战",
 * section "核心代码解析", MoEOperator::Forward):
 *
 *   logits = x @ W_router (+ gate_bias)             gate GEMM
 *   p      = softmax(logits)                          per token, over E experts
 *   idx, w = top-k of p, renormalised over the k      lower expert index wins ties
 *            (or, threshold routing: the experts with p > delta, at most k of them)
 *   rows   = tokens grouped by expert, token order    capacity clamp, then gather
 *   h      = silu(x_e Wg[e]) * (x_e Wu[e])            grouped GEMM 1 (GELU: gelu(x_e Wu[e]))
 *   y      = h Wd[e]                                  grouped GEMM 2
 *   out[t] = sum_j w[t,j] * y[row(t,j)]               combine, one write per row, no atomics
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a device pointer owned by the caller; the library never
 *     allocates, frees or keeps a pointer after returning. All scratch memory comes from
 *     the caller's workspace `ws` of `ws_bytes` bytes (size it with moe_workspace_size);
 *     it is sized for the worst case of T*k routed rows, so no routing outcome can
 *     overflow it.
 *   - Layouts are dense and row-major: x[T,H], W_router[H,E], W_gate/W_up[E,H,I],
 *     W_down[E,I,H] (the pages' x[tokens,hidden] and expert weights
 *     [num_experts,hidden,intermediate]: lshu.cn/news/82007, section 3). Element type is
 *     cfg->dtype for x, the weights, x_perm, h, y_perm and out; logits and gate weights
 *     are float32; expert ids and row indices are int32 (lshu.cn page, section 5.2).
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL is the null stream), do no
 *     device->host synchronisation (moe_read_device_status excepted) and keep no global
 *     mutable state (moe_permute_noalloc's fixed scratch excepted), so they are safe to
 *     call from several host threads. Calls that share one workspace must be ordered on one
 *     stream.
 *   - Alignment: every tensor of the layer dtype (x, w_router in bf16, w_gate, w_up,
 *     w_down and their packed forms, x_perm, h, y_perm, out, dout, dx and the weight
 *     gradients) and the workspaces ws / bws must be 16-byte aligned, since the kernels move
 *     them in 16-byte pieces; float32 and int32 arrays (logits, gate weights and bias, ids,
 *     row maps, counts, offsets, dw_router) need 4 bytes, and an fp32 w_router 4 bytes.
 *     A pointer that breaks this is MOE_ERR_INVALID_ARG.
 *   - Argument errors are reported synchronously, before any HIP call, as a moe_status;
 *     nothing aborts or prints. A failed kernel launch returns MOE_ERR_HIP and the HIP
 *     error code is kept per host thread (moe_last_hip_error).
 *   - Data errors found on the device (an expert id outside [0,E) or repeated within a
 *     token, a non-finite logit) never cause an out-of-bounds access: the offending slot
 *     is dropped and a flag is raised, to be read with moe_read_device_status. Ids are
 *     never clamped silently.
 *   - tokens == 0 is a valid empty call: once the configuration is valid, MOE_OK is
 *     returned without inspecting any pointer and nothing is launched.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size, k outside [1, E] ... */
  MOE_ERR_UNSUPPORTED = 2,   /* valid but not supported: E or k above the maximum, a dtype /
                                activation value outside the enums, bf16 sizes that are not
                                multiples of the GEMM tiles */
  MOE_ERR_WORKSPACE = 3,     /* ws_bytes smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4            /* a HIP call or kernel launch failed */
} moe_status;

enum { MOE_DTYPE_BF16 = 0, MOE_DTYPE_F32 = 1 };
enum { MOE_ACT_SWIGLU = 0, MOE_ACT_GELU = 1 };
/* device status flags (moe_read_device_status) */
enum { MOE_FLAG_BAD_INDEX = 1, MOE_FLAG_NONFINITE_LOGIT = 2, MOE_FLAG_STALE_SAVED = 4 };
enum { MOE_MAX_EXPERTS = 256, MOE_MAX_TOPK = 16 };
/* routing rules (moe_config.routing) */
enum { MOE_ROUTE_TOPK = 0, MOE_ROUTE_THRESHOLD = 1 };
/* weight layouts (moe_config.weight_layout, bit flags) and weights (moe_pack_expert_weight) */
enum { MOE_WEIGHTS_PLAIN = 0, MOE_WEIGHTS_PACKED = 1, MOE_ROUTER_PACKED = 2 };
enum { MOE_WEIGHT_GATE = 0, MOE_WEIGHT_UP = 1, MOE_WEIGHT_DOWN = 2, MOE_WEIGHT_ROUTER = 3 };

typedef struct moe_config {
  int32_t tokens;            /* T >= 0 */
  int32_t hidden;            /* H >= 1; bf16: multiple of 256 */
  int32_t inter;             /* I >= 1; bf16: multiple of 128 (SwiGLU), 256 (GELU) */
  int32_t experts;           /* E in [1, MOE_MAX_EXPERTS] */
  int32_t top_k;             /* k in [1, min(E, MOE_MAX_TOPK)] */
  int32_t activation;        /* MOE_ACT_SWIGLU or MOE_ACT_GELU */
  int32_t dtype;             /* MOE_DTYPE_BF16 or MOE_DTYPE_F32 (f32: H multiple of 8) */
  int32_t renormalize;       /* nonzero: weights renormalised over the k selected experts
                                (mhpn.cn/news/871594 chapter 8, normalize_scores=True);
                                zero: the raw softmax probabilities (intelliparadigm.com
                                page, section 2.1) */
  double capacity_factor;    /* <= 0: no limit. Otherwise each expert keeps at most
                                C = ceil(capacity_factor * (T*k) / E) assignments, lowest
                                token index first (hnwysp.cn/news/132341, section 3.2) */
  int32_t routing;           /* MOE_ROUTE_TOPK (0, the default): the k best experts.
                                MOE_ROUTE_THRESHOLD: every expert whose softmax score p
                                exceeds `threshold` (strictly, decided in float64), best
                                first, at most top_k of them; unused slots get id -1 and
                                weight 0, and a token with none above the threshold
                                contributes zero (intelliparadigm.com page, section 3.2.1:
                                keep the experts scoring above delta, default 1/E, then
                                renormalise) */
  int32_t weight_layout;     /* bit flags; MOE_WEIGHTS_PLAIN (0, the default): every weight
                                in the row-major layouts below. MOE_WEIGHTS_PACKED (bf16
                                only): w_gate, w_up, w_down as written by
                                moe_pack_expert_weight, for the forward entry points
                                (moe_expert_up, moe_expert_up_rows, moe_expert_down,
                                moe_grouped_ffn, moe_forward). MOE_ROUTER_PACKED (bf16
                                only): w_router as written by moe_pack_expert_weight
                                (MOE_WEIGHT_ROUTER), for moe_route and moe_forward. The
                                backward and moe_forward_train need plain weights (either
                                bit: MOE_ERR_UNSUPPORTED). Other bits: MOE_ERR_INVALID_ARG */
  double threshold;          /* delta of MOE_ROUTE_THRESHOLD; <= 0 means 1/E; not NaN */
  double aux_loss_coeff;     /* >= 0, not NaN. > 0: moe_backward also differentiates the
                                auxiliary load-balancing loss coeff * E * sum_e f_e P_e (f_e:
                                fraction of the routed assignments, before capacity, that
                                chose expert e; P_e: mean softmax probability of e over the
                                tokens) and leaves its value in the MOE_WS_AUX_LOSS view. The
                                pages add such a loss term to balance the experts' load
                                (mhpn.cn/news/871594, routing chapter), with MindSpeed's
                                moe-aux-loss-coeff 0.01, at most 0.1 (lshu.cn/news/82007,
                                section 5.3), but give no formula; this is the switch-style
                                one. 0 (the default): off */
} moe_config;

typedef void* moe_stream_t;  /* hipStream_t */

/* Workspace bytes needed by every entry point below for this configuration. */
moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes);

/* The capacity C the kernels use: ceil(cf * (T*k) / E) evaluated in IEEE double, or T
 * when cf <= 0. */
moe_status moe_capacity(const moe_config* cfg, int32_t* capacity);

/* Gate GEMM + softmax + top-k + weights (gitcode page, "核心代码解析": routing_module_,
 * TopKRouting; hnwysp.cn page, section 2.1: top-k routing; section 4.1: softmax first).
 *   x         [T,H] dtype, or NULL: then `logits` is an INPUT and only top-k runs
 *   w_router  [H,E] dtype, or with MOE_ROUTER_PACKED in weight_layout the same weight as
 *             written by moe_pack_expert_weight (MOE_WEIGHT_ROUTER; 16-byte aligned);
 *             ignored when x == NULL. The two give bit-identical results
 *   gate_bias [E] float32 or NULL, added to the logits before softmax and selection
 *   logits    [T,E] float32: output (input when x == NULL)
 *   topk_idx  [T,k] int32 out: experts in descending logit order, lower index first on ties
 *             (threshold routing: the kept experts in that order, then -1)
 *   topk_w    [T,k] float32 out: softmax weights of those experts (renormalised if set);
 *             NaN for a token with a NaN logit (threshold routing: 0 in unused slots; a
 *             token with a NaN or +inf logit keeps no expert)
 * Non-finite logits raise MOE_FLAG_NONFINITE_LOGIT; NaN ranks below -inf. */
moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* gate_bias, float* logits, int32_t* topk_idx, float* topk_w,
                     void* ws, size_t ws_bytes, moe_stream_t stream);

/* Histogram + scan + capacity clamp + gather of token rows by expert (gitcode page,
 * SparseGather and the CSR storage of "MoE 算子核心原理"; lshu.cn page, section 4,
 * npu_moe_token_preprocess).
 *   x              [T,H] dtype
 *   topk_idx       [T,k] int32 expert ids; -1 is an empty slot (dropped, no flag); any
 *                  other id outside [0,E), or a repeat within a token, is dropped + flagged
 *   x_perm         [T*k,H] dtype out: rows grouped by expert, token order inside an expert;
 *                  rows >= expert_offsets[E] are left untouched. May be NULL: then only the
 *                  row maps below are written (x is not read), for moe_expert_up_rows
 *   expert_counts  [E] int32 out: assignments per expert before the capacity clamp
 *   expert_offsets [E+1] int32 out: first row of each expert after the clamp
 *   row_token      [T*k] int32 out: source token of each row (rows < expert_offsets[E])
 *   slot_row       [T,k] int32 out: row of slot (t,j), -1 if dropped or invalid */
moe_status moe_permute(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                       void* x_perm, int32_t* expert_counts, int32_t* expert_offsets,
                       int32_t* row_token, int32_t* slot_row, void* ws, size_t ws_bytes,
                       moe_stream_t stream);

/* moe_route followed by moe_permute's row maps (x_perm NULL), as moe_forward runs them,
 * with the same arguments, meanings and results, bit for bit (gitcode page, routing_module_
 * then SparseGather's per-expert grouping; lshu.cn page, section 4, the token reordering
 * after routing). For a bf16 gate of at most 16 experts (the streaming router) the
 * permutation's count step runs inside the router and the whole takes two launches
 * instead of three; otherwise it is the two calls one after the other. The device flags
 * of both steps land where moe_read_device_status reads them (which = 1 and 2).
 *   x may be NULL (logits an INPUT), as for moe_route */
moe_status moe_route_permute(const moe_config* cfg, const void* x, const void* w_router,
                             const float* gate_bias, float* logits, int32_t* topk_idx,
                             float* topk_w, int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* row_token, int32_t* slot_row, void* ws, size_t ws_bytes,
                             moe_stream_t stream);

/* moe_permute for callers that cannot allocate device memory or hand over a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same results as moe_permute, bit for bit, with its scratch (the per-block expert
 * histograms and flags) in a fixed device array inside the library instead of `ws`. It
 * calls no allocating routine. The array is MOE_NOALLOC_SCRATCH_BYTES per device (each
 * device that runs this call holds its own copy until the process ends) and this call uses
 * ceil(T / 1024) * (E + 1) * 4 bytes of it: a larger T or E -> MOE_ERR_WORKSPACE, before any
 * HIP call. Every call on one device shares that device's array, so calls that overlap on
 * one device (different streams, or different host threads) race: order them on one
 * stream. The stream must belong to the current device; the array's device address is
 * looked up once per device, on the first call there (the library's only global state,
 * guarded for concurrent first calls).
 *   x, topk_idx, x_perm (or NULL), expert_counts, expert_offsets, row_token, slot_row:
 *       as for moe_permute
 *   flags  [1] int32 out, or NULL: the device flags moe_permute would raise
 *          (MOE_FLAG_BAD_INDEX), since no workspace holds them for moe_read_device_status */
enum { MOE_NOALLOC_SCRATCH_BYTES = 1 << 20 };
moe_status moe_permute_noalloc(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                               void* x_perm, int32_t* expert_counts, int32_t* expert_offsets,
                               int32_t* row_token, int32_t* slot_row, int32_t* flags,
                               moe_stream_t stream);

/* Grouped GEMM 1 with the activation fused: for the rows of each expert e,
 * h = silu(x_perm Wg[e]) * (x_perm Wu[e])  (SwiGLU)   or   h = gelu(x_perm Wu[e])  (GELU)
 * (lshu.cn page, section 3: npu_moe_final_optimizer_mm is this up-projection; the
 * activation and the down-projection follow it).
 *   x_perm [rows,H], expert_offsets [E+1] (device; values are clamped to [0, T*k] and an
 *   empty or reversed range counts as empty), w_gate [E,H,I] (NULL for GELU),
 *   w_up [E,H,I], h [T*k,I] out (rows >= expert_offsets[E] untouched). */
moe_status moe_expert_up(const moe_config* cfg, const void* x_perm,
                         const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                         void* h, moe_stream_t stream);

/* Grouped GEMM 1 with the permute gather fused into its operand loads: as moe_expert_up,
 * but row r of the expert-major operand is read in place as token row x[row_token[r]]
 * instead of from a materialised x_perm (lshu.cn/news/82007, section 1: the case for fusing
 * the token permutation with the expert matmul; section 3, the fused up-projection).
 *   x         [T,H] dtype, the token rows (not permuted)
 *   row_token [T*k] int32, source token of each row, as written by moe_permute; entries
 *             outside [0, T) are clamped into it (never read out of bounds)
 *   expert_offsets, w_gate, w_up, h as for moe_expert_up.
 * h is bit-identical to moe_expert_up on the x_perm that moe_permute would produce. */
moe_status moe_expert_up_rows(const moe_config* cfg, const void* x, const int32_t* row_token,
                              const int32_t* expert_offsets, const void* w_gate,
                              const void* w_up, void* h, moe_stream_t stream);

/* Grouped GEMM 2: y_perm = h Wd[e] for the rows of each expert (lshu.cn page, section 4,
 * npu_moe_matmul). h [rows,I], w_down [E,I,H], y_perm [T*k,H] out.
 * ws / ws_bytes: the layer's workspace (at least moe_workspace_size bytes), or NULL. With a
 * workspace, bf16 layers run the tiles left over after the last whole round of the grid as
 * K slices over all CUs (float32 partials in ws, added in a fixed order by a second kernel on
 * the same stream), so y_perm stays deterministic; without one, every tile runs whole. The
 * two differ only in float32 summation order. ws too small -> MOE_ERR_WORKSPACE. */
moe_status moe_expert_down(const moe_config* cfg, const void* h, const int32_t* expert_offsets,
                           const void* w_down, void* y_perm, void* ws, size_t ws_bytes,
                           moe_stream_t stream);

/* moe_expert_up followed by moe_expert_down, with h kept in the workspace. */
moe_status moe_grouped_ffn(const moe_config* cfg, const void* x_perm,
                           const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                           const void* w_down, void* y_perm, void* ws, size_t ws_bytes,
                           moe_stream_t stream);

/* Repack one weight tensor for MOE_WEIGHTS_PACKED or MOE_ROUTER_PACKED (bf16 only; once,
 * when weights are loaded: inference weights are constant; the pages likewise store their
 * weights in the matrix unit's own NZ format, lshu.cn page, section 5.1). `packed` must
 * hold moe_packed_weight_bytes(cfg, which) bytes, be 16-byte aligned and not overlap w.
 *   which = MOE_WEIGHT_GATE or MOE_WEIGHT_UP (w [E,H,I]; gate: SwiGLU only) or
 *   MOE_WEIGHT_DOWN (w [E,I,H]): for w [E,K,N], `packed` (the same byte size) receives, for
 *   each expert e, 32-column block nb and 16-row slice ks, a 1 KB block whose 16-byte chunk
 *   l (0..63) holds
 *     w[e][16 ks + 8 (l >> 5) + q][32 nb + (l & 31)],  q = 0..7,
 *   blocks ordered [e][nb][ks]: chunk l is lane l's operand of one 32x32x16 bf16 MFMA, so
 *   the packed GEMMs load weights straight into registers.
 *   which = MOE_WEIGHT_ROUTER (w = w_router [H,E]): `packed` receives, for each group g of
 *   16 experts (EP / 16 groups, EP the smallest of 32, 64, 128, 256 that is >= E) and
 *   32-row slice s, a 1 KB block whose 16-byte chunk l holds
 *     w[32 s + 8 (l >> 4) + q][16 g + (l & 15)],  q = 0..7 (0 for experts >= E),
 *   blocks ordered [g][s]: lane l's operand of one 16x16x32 bf16 MFMA of the gate GEMM.
 * Results with packed weights are bit-identical to plain ones (the summation order is
 * unchanged). Asynchronous on `stream`; a bad `which` or overlapping buffers ->
 * MOE_ERR_INVALID_ARG. */
moe_status moe_pack_expert_weight(const moe_config* cfg, int32_t which, const void* w,
                                  void* packed, moe_stream_t stream);

/* Bytes of moe_pack_expert_weight's output for `which` (0 for a bad which or config):
 * E*H*I*2 for the expert weights, EP*H*2 for the router. */
size_t moe_packed_weight_bytes(const moe_config* cfg, int32_t which);

/* Weighted combine back to token order (lshu.cn page, section 4,
 * npu_moe_token_postprocess; the pages aggregate with an atomic scatter-add, this library
 * gathers instead): out[t] = sum over kept slots of topk_w[t,j] * y_perm[slot_row[t,j]]
 * (a slot is kept when 0 <= slot_row[t,j] < T*k),
 * accumulated in float32 in slot order and written once per row; a token whose slots were
 * all dropped gets zeros. y_perm [rows,H], slot_row [T,k], topk_w [T,k], out [T,H]. */
moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* slot_row,
                       const float* topk_w, void* out, moe_stream_t stream);

/* The whole layer: moe_route -> the row maps of moe_permute -> moe_expert_up_rows (the
 * gather fused into GEMM 1, so x_perm is never materialised) -> moe_expert_down ->
 * moe_combine, with every intermediate in `ws` (readable with moe_workspace_view until the
 * next call). */
moe_status moe_forward(const moe_config* cfg, const void* x, const void* w_router,
                       const float* gate_bias, const void* w_gate, const void* w_up,
                       const void* w_down, void* out, void* ws, size_t ws_bytes,
                       moe_stream_t stream);

/* Backward pass of the layer: the gradients of sum(out * dout) with respect to x, the router
 * weight, the gate bias and the expert weights (gitcode page, "MoE 算子核心原理": the
 * backward runs on the selected experts only). The expert choice (top-k, threshold,
 * capacity) carries no gradient; the gate weights' dependence on the logits is exact. With
 * cfg->aux_loss_coeff > 0 the auxiliary load-balancing loss is added to that objective: its
 * logit gradient p (g - <p, g>), g_e = coeff * E * f_e / T, joins the router's before dx,
 * dw_router and dgate_bias are formed, and its value (float64) is written to the
 * MOE_WS_AUX_LOSS view of `ws`.
 *   ws, ws_bytes   the workspace of a moe_forward (or moe_forward_train) call with the same
 *                  cfg, x and weights, made on the same stream before this call: its
 *                  routing, row maps and y_perm are reused (so is its gate bias, through the
 *                  logits)
 *   bws, bws_bytes backward scratch, at least moe_backward_workspace_size bytes
 *   saved          nonzero: that call was moe_forward_train with this bws, which kept the
 *                  up-projection's pre-activations there; zero: they are recomputed here.
 *                  Precondition of saved != 0: no other call built a permutation in ws
 *                  after that moe_forward_train (moe_forward, moe_forward_train,
 *                  moe_permute). Every permutation advances a generation counter in ws
 *                  and moe_forward_train records its value in bws; when they differ the
 *                  backward raises MOE_FLAG_STALE_SAVED (moe_read_device_status, which = 4)
 *                  and its gradients are not to be used
 *   dout [T,H] bf16 in; dx [T,H] bf16 out; dw_router [H,E] float32 out; dgate_bias [E]
 *   float32 out or NULL; dw_gate (SwiGLU only; NULL for GELU), dw_up [E,H,I] and dw_down
 *   [E,I,H] bf16 out (float32 accumulation, rounded once)
 * bf16 layers with I a multiple of 256 only (else MOE_ERR_UNSUPPORTED). Expert rows are
 * regrouped in a padded row space (each expert's rows rounded up to a multiple of 128); with
 * saved = 0 the up-projection is recomputed there. */
moe_status moe_backward_workspace_size(const moe_config* cfg, size_t* bytes);
moe_status moe_backward(const moe_config* cfg, const void* x, const void* w_router,
                        const void* w_gate, const void* w_up, const void* w_down,
                        const void* dout, void* dx, float* dw_router, float* dgate_bias,
                        void* dw_gate, void* dw_up, void* dw_down, void* ws, size_t ws_bytes,
                        void* bws, size_t bws_bytes, int32_t saved, moe_stream_t stream);

/* moe_forward for training: the same output, and GEMM 1 also keeps its pre-activations
 * ([g | u] per kept row; GELU: a) in `bws` for a following moe_backward(..., saved = 1), which
 * then skips recomputing the up-projection. Same arguments as moe_forward plus the backward
 * scratch; bf16 layers with I a multiple of 256 (else MOE_ERR_UNSUPPORTED). */
moe_status moe_forward_train(const moe_config* cfg, const void* x, const void* w_router,
                             const float* gate_bias, const void* w_gate, const void* w_up,
                             const void* w_down, void* out, void* ws, size_t ws_bytes,
                             void* bws, size_t bws_bytes, moe_stream_t stream);

/* Where moe_forward keeps an intermediate inside `ws` (device address and byte size). */
enum {
  MOE_WS_LOGITS = 0,      /* [T,E] float32 */
  MOE_WS_TOPK_IDX = 1,    /* [T,k] int32 */
  MOE_WS_TOPK_W = 2,      /* [T,k] float32 */
  MOE_WS_COUNTS = 3,      /* [E] int32 */
  MOE_WS_OFFSETS = 4,     /* [E+1] int32 */
  MOE_WS_SLOT_ROW = 5,    /* [T,k] int32 */
  MOE_WS_ROW_TOKEN = 6,   /* [T*k] int32 */
  MOE_WS_X_PERM = 7,      /* not materialised by moe_forward: view -> MOE_ERR_INVALID_ARG */
  MOE_WS_H = 8,           /* [T*k,I] dtype */
  MOE_WS_Y_PERM = 9,      /* [T*k,H] dtype */
  MOE_WS_AUX_LOSS = 10,   /* [1] float64: the auxiliary load-balancing loss, written by a
                             moe_backward with aux_loss_coeff > 0 */
  MOE_WS_NUM_VIEWS = 11
};
moe_status moe_workspace_view(const moe_config* cfg, void* ws, int32_t which, void** dev_ptr,
                              size_t* bytes);

/* OR of the device flags raised by the last moe_route (which bit 1), the last moe_permute
 * (bit 2) and the last moe_backward (bit 4: MOE_FLAG_STALE_SAVED) that used this workspace;
 * which in [1, 7] selects any mix of them (moe_forward runs route and permute).
 * Synchronises `stream`. */
moe_status moe_read_device_status(const moe_config* cfg, void* ws, int32_t which,
                                  moe_stream_t stream, int32_t* flags);

const char* moe_status_string(moe_status status);
int32_t moe_last_hip_error(void);   /* hipError_t of this thread's last MOE_ERR_HIP */

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
