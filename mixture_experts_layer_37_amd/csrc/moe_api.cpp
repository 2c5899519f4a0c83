// Host side of the C ABI declared in include/moe.h: argument validation (before any HIP
// call), workspace layout, the capacity formula and the launch sequence on the caller's
// stream. No allocation, no global mutable state apart from the per-thread last HIP error.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstddef>
#include <cmath>
#include <cstring>
#include <vector>

#include "moe.h"
#include "kernels.h"

// The binding mirrors this layout (explicit 32-bit fields, no implicit padding).
static_assert(MOE_NOALLOC_SCRATCH_BYTES == moe::kNoAllocScratchWords * 4,
              "the header states the size of the no-allocation scratch");
static_assert(sizeof(moe_config) == 64 && offsetof(moe_config, routing) == 40 &&
                  offsetof(moe_config, weight_layout) == 44 &&
                  offsetof(moe_config, threshold) == 48 &&
                  offsetof(moe_config, aux_loss_coeff) == 56,
              "moe_config layout");

namespace {

thread_local int g_last_hip_error = 0;

enum Region {
  R_WT, R_LOGITS, R_TOPK_IDX, R_TOPK_W, R_ROUTE_FLAGS, R_HIST, R_PERM_FLAGS, R_COUNTS,
  R_OFFSETS, R_SLOT_ROW, R_ROW_TOKEN, R_H, R_Y_PERM, R_SPLIT, R_AUX_LOSS, R_GEN, R_NUM
};

struct Layout {
  size_t off[R_NUM];
  size_t size[R_NUM];
  size_t total;
};

constexpr size_t kAlign = 256;

size_t esize(const moe_config* c) { return c->dtype == MOE_DTYPE_BF16 ? 2 : 4; }

// Whether route and permute run as two launches (moe_route_permute, moe_forward): the
// streaming router counts the permutation's assignments itself, per block of 32 tokens.
bool routed_count(const moe_config* c) {
  return c->dtype == MOE_DTYPE_BF16 && moe::route_lds_fits(c->hidden, c->experts) &&
         (c->tokens + moe::kRouteCountTokens - 1) / moe::kRouteCountTokens <=
             moe::kRoutedMaxBlocks;
}

Layout layout_of(const moe_config* c) {
  const size_t T = (size_t)c->tokens, H = (size_t)c->hidden, I = (size_t)c->inter;
  const size_t E = (size_t)c->experts, k = (size_t)c->top_k, es = esize(c);
  const size_t N = T * k;
  const size_t NB = (size_t)moe::permute_count_blocks(c->tokens);
  Layout L;
  L.size[R_WT] = (c->dtype == MOE_DTYPE_BF16 && !moe::route_lds_fits(c->hidden, c->experts))
                    ? (size_t)moe::route_padded_experts(c->experts) * H * 2
                    : 0;
  L.size[R_LOGITS] = T * E * 4;
  L.size[R_TOPK_IDX] = N * 4;
  L.size[R_TOPK_W] = N * 4;
  L.size[R_ROUTE_FLAGS] = ((T + moe::kRouteFlagGroup - 1) / moe::kRouteFlagGroup) * 4;
  // the count kernel's histogram table, or the router's (one row per 32 tokens)
  const size_t NBR = (T + moe::kRouteCountTokens - 1) / moe::kRouteCountTokens;
  L.size[R_HIST] = (routed_count(c) ? NBR : NB) * E * 4;
  L.size[R_PERM_FLAGS] = NB * 4;
  L.size[R_COUNTS] = E * 4;
  L.size[R_OFFSETS] = (E + 1) * 4;
  L.size[R_SLOT_ROW] = N * 4;
  L.size[R_ROW_TOKEN] = N * 4;
  L.size[R_H] = N * I * es;
  L.size[R_Y_PERM] = N * H * es;
  // float32 partial tiles of GEMM 2's split-K tail (bf16 path)
  L.size[R_SPLIT] = c->dtype == MOE_DTYPE_BF16 ? moe::kSplitPartialBytes : 0;
  L.size[R_AUX_LOSS] = 8;   // float64
  // [0] permutation generation (advanced by every permutation built in this workspace),
  // [1] backward flags (MOE_FLAG_STALE_SAVED)
  L.size[R_GEN] = 8;
  size_t o = 0;
  for (int r = 0; r < R_NUM; ++r) {
    L.off[r] = o;
    o += (L.size[r] + kAlign - 1) / kAlign * kAlign;
  }
  L.total = o;
  return L;
}

template <typename P> P* region(void* ws, const Layout& L, Region r) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + L.off[r]);
}

// ---- backward workspace: the padded row space of the backward (multiples of 128 rows per
// expert), the recomputed activations and the gradients on their way.
enum BRegion {
  B_POFF, B_PROW, B_XP, B_GU, B_H, B_DY, B_DGU, B_DXP, B_DL, B_DW, B_SPLIT, B_WRPART, B_BPART,
  B_XPK, B_DYPK, B_AUXP, B_AUXG, B_GEN, B_NUM
};

struct BLayout {
  size_t off[B_NUM];
  size_t size[B_NUM];
  size_t total;
};

BLayout blayout_of(const moe_config* c) {
  BLayout L{};
  const size_t T = (size_t)c->tokens, H = (size_t)c->hidden, I = (size_t)c->inter;
  const size_t E = (size_t)c->experts, k = (size_t)c->top_k;
  const size_t P = (size_t)moe::bwd_padded_rows(c->tokens, c->top_k, c->experts);
  const size_t pair = c->activation == MOE_ACT_SWIGLU ? 2 : 1;   // [g | u] or a
  L.size[B_POFF] = (E + 1) * 4;
  L.size[B_PROW] = P * 4;
  L.size[B_XP] = P * H * 2;
  L.size[B_GU] = P * pair * I * 2;
  L.size[B_H] = P * I * 2;
  L.size[B_DY] = P * H * 2;
  L.size[B_DGU] = P * pair * I * 2;
  L.size[B_DXP] = P * H * 2;
  L.size[B_DL] = T * E * 4;
  L.size[B_DW] = T * k * 4;
  L.size[B_SPLIT] = moe::kSplitPartialBytes;
  L.size[B_WRPART] = (size_t)moe::bwd_wrouter_chunks(c->tokens) * H * E * 4;
  L.size[B_BPART] = (size_t)moe::bwd_wrouter_chunks(c->tokens) * E * 4;
  // x rows and dy in the packed operand layout, for the weight gradients' register operand
  L.size[B_XPK] = (P / 16) * 16 * H * 2;
  L.size[B_DYPK] = (P / 16) * 16 * H * 2;
  // auxiliary load-balancing loss: per-block probability sums and per-expert gradients
  L.size[B_AUXP] = c->aux_loss_coeff > 0 ? (size_t)moe::bwd_aux_blocks(c->tokens) * E * 8 : 0;
  L.size[B_AUXG] = c->aux_loss_coeff > 0 ? E * 8 : 0;
  // the workspace generation of the training forward whose pre-activations B_GU holds
  L.size[B_GEN] = 4;
  size_t o = 0;
  for (int r = 0; r < B_NUM; ++r) {
    L.off[r] = o;
    o += (L.size[r] + kAlign - 1) / kAlign * kAlign;
  }
  L.total = o;
  return L;
}

template <typename P> P* bregion(void* ws, const BLayout& L, BRegion r) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + L.off[r]);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

moe_status check_cfg(const moe_config* c) {
  if (c == nullptr) return MOE_ERR_INVALID_ARG;
  if (c->tokens < 0 || c->hidden < 1 || c->inter < 1 || c->experts < 1 || c->top_k < 1)
    return MOE_ERR_INVALID_ARG;
  if (c->top_k > c->experts) return MOE_ERR_INVALID_ARG;
  if (std::isnan(c->capacity_factor)) return MOE_ERR_INVALID_ARG;
  if (c->routing != MOE_ROUTE_TOPK && c->routing != MOE_ROUTE_THRESHOLD)
    return MOE_ERR_INVALID_ARG;
  if (std::isnan(c->threshold)) return MOE_ERR_INVALID_ARG;
  if (!(c->aux_loss_coeff >= 0.0) || std::isinf(c->aux_loss_coeff)) return MOE_ERR_INVALID_ARG;
  if ((c->weight_layout & ~(MOE_WEIGHTS_PACKED | MOE_ROUTER_PACKED)) != 0)
    return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_DTYPE_BF16 && c->dtype != MOE_DTYPE_F32) return MOE_ERR_UNSUPPORTED;
  if (c->weight_layout != MOE_WEIGHTS_PLAIN && c->dtype != MOE_DTYPE_BF16)
    return MOE_ERR_UNSUPPORTED;
  if (c->activation != MOE_ACT_SWIGLU && c->activation != MOE_ACT_GELU) return MOE_ERR_UNSUPPORTED;
  if (c->experts > MOE_MAX_EXPERTS || c->top_k > MOE_MAX_TOPK) return MOE_ERR_UNSUPPORTED;
  if (c->dtype == MOE_DTYPE_BF16) {
    if (c->hidden % 256 != 0) return MOE_ERR_UNSUPPORTED;
    if (c->inter % (c->activation == MOE_ACT_SWIGLU ? 128 : 256) != 0) return MOE_ERR_UNSUPPORTED;
  } else if (c->hidden % 8 != 0) {
    return MOE_ERR_UNSUPPORTED;
  }
  const long long T = c->tokens, k = c->top_k;
  const long long wide = (long long)(c->hidden > c->inter ? c->hidden : c->inter);
  if (T * k > INT_MAX || T * c->experts > INT_MAX || T * k * wide > (1LL << 40))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int capacity_of(const moe_config* c) {
  if (!(c->capacity_factor > 0.0)) return c->tokens;
  const double v = std::ceil((c->capacity_factor * (double)((long long)c->tokens * c->top_k)) /
                             (double)c->experts);
  return v >= (double)INT_MAX ? INT_MAX : (int)v;
}

moe_status hip_status(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  g_last_hip_error = (int)e;
  return MOE_ERR_HIP;
}

#define MOE_TRY(expr)                              \
  do {                                             \
    const moe_status st_ = (expr);                 \
    if (st_ != MOE_OK) return st_;                 \
  } while (0)

moe_status check_ws(const moe_config* c, void* ws, size_t ws_bytes) {
  if (ws == nullptr || !aligned(ws, 16)) return MOE_ERR_INVALID_ARG;
  if (ws_bytes < layout_of(c).total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

// The backward's tiles: bf16 only, I a multiple of 256 (256-wide gradient tiles over I),
// plain weights (its products read them transposed in place).
moe_status check_backward_cfg(const moe_config* c) {
  MOE_TRY(check_cfg(c));
  if (c->dtype != MOE_DTYPE_BF16 || c->inter % 256 != 0) return MOE_ERR_UNSUPPORTED;
  if (c->weight_layout != MOE_WEIGHTS_PLAIN) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status need(const void* p, size_t align) {
  return (p != nullptr && aligned(p, align)) ? MOE_OK : MOE_ERR_INVALID_ARG;
}

// ---- the steps, arguments already validated
moe_status do_route(const moe_config* c, const void* x, const void* w_router, const float* bias,
                    float* logits, int32_t* idx, float* w, void* ws, hipStream_t s) {
  const Layout L = layout_of(c);
  int32_t* flags = region<int32_t>(ws, L, R_ROUTE_FLAGS);
  const int T = c->tokens, H = c->hidden, E = c->experts, k = c->top_k;
  const int renorm = c->renormalize != 0;
  // threshold routing: delta (<= 0 means 1/E), compared in float64
  const int thr = c->routing == MOE_ROUTE_THRESHOLD;
  const double delta = c->threshold > 0 ? c->threshold : 1.0 / (double)E;
  if (x == nullptr)
    return hip_status(
        moe::launch_route_topk(logits, idx, w, flags, T, E, k, renorm, thr, delta, s));
  // a router weight packed at load time (MOE_ROUTER_PACKED) is already in the MFMA operand
  // order the routers read; a plain one goes to the streaming router as it is, or is
  // packed into the workspace for the general router
  const bool packed = (c->weight_layout & MOE_ROUTER_PACKED) != 0;
  if (c->dtype == MOE_DTYPE_BF16 && moe::route_lds_fits(H, E))
    return hip_status(moe::launch_route_bf16_lds(
        (const moe::bf16_t*)x, packed ? nullptr : (const moe::bf16_t*)w_router,
        packed ? (const moe::bf16_t*)w_router : nullptr, bias, logits, idx, w, flags, nullptr,
        nullptr, T, H, E, k, renorm, thr, delta, moe::device_cus(), s));
  if (c->dtype == MOE_DTYPE_BF16) {
    const moe::bf16_t* wt = (const moe::bf16_t*)w_router;
    if (!packed) {
      moe::bf16_t* wp = region<moe::bf16_t>(ws, L, R_WT);
      MOE_TRY(hip_status(moe::launch_router_pack((const moe::bf16_t*)w_router, wp, H, E, s)));
      wt = wp;
    }
    return hip_status(moe::launch_route_bf16((const moe::bf16_t*)x, wt, bias, logits, idx, w,
                                             flags, T, H, E, k, renorm, thr, delta, s));
  }
  MOE_TRY(hip_status(moe::launch_route_logits_f32((const float*)x, (const float*)w_router, bias,
                                                  logits, T, H, E, s)));
  return hip_status(
      moe::launch_route_topk(logits, idx, w, flags, T, E, k, renorm, thr, delta, s));
}

// gen_copy (may be null): where a training forward records the new permutation generation
moe_status do_permute(const moe_config* c, const void* x, const int32_t* idx, void* x_perm,
                      int32_t* counts, int32_t* offsets, int32_t* row_token, int32_t* slot_row,
                      void* ws, hipStream_t s, int32_t* gen_copy = nullptr) {
  const Layout L = layout_of(c);
  const int cap = capacity_of(c);
  return hip_status(moe::launch_permute(
      x, (int)esize(c), idx, x_perm, counts, offsets, row_token, slot_row,
      region<int32_t>(ws, L, R_HIST), region<int32_t>(ws, L, R_PERM_FLAGS),
      region<int32_t>(ws, L, R_GEN), gen_copy, nullptr, c->tokens, c->hidden, c->experts,
      c->top_k, cap < c->tokens ? cap : c->tokens, s));
}

// Route, then the permutation's row maps (no x_perm). With the streaming router the count
// step runs in the router's epilogue and one more launch builds the maps; otherwise the
// two steps as moe_route and moe_permute run them. Same results either way.
moe_status do_route_permute(const moe_config* c, const void* x, const void* w_router,
                            const float* bias, float* logits, int32_t* idx, float* w,
                            int32_t* counts, int32_t* offsets, int32_t* row_token,
                            int32_t* slot_row, void* ws, hipStream_t s,
                            int32_t* gen_copy = nullptr) {
  if (x == nullptr || !routed_count(c)) {
    MOE_TRY(do_route(c, x, w_router, bias, logits, idx, w, ws, s));
    return do_permute(c, x, idx, nullptr, counts, offsets, row_token, slot_row, ws, s,
                      gen_copy);
  }
  const Layout L = layout_of(c);
  const int T = c->tokens, H = c->hidden, E = c->experts, k = c->top_k;
  const int thr = c->routing == MOE_ROUTE_THRESHOLD;
  const double delta = c->threshold > 0 ? c->threshold : 1.0 / (double)E;
  const bool packed = (c->weight_layout & MOE_ROUTER_PACKED) != 0;
  int32_t* hist = region<int32_t>(ws, L, R_HIST);
  MOE_TRY(hip_status(moe::launch_route_bf16_lds(
      (const moe::bf16_t*)x, packed ? nullptr : (const moe::bf16_t*)w_router,
      packed ? (const moe::bf16_t*)w_router : nullptr, bias, logits, idx, w,
      region<int32_t>(ws, L, R_ROUTE_FLAGS), hist, slot_row, T, H, E, k, c->renormalize != 0,
      thr, delta, moe::device_cus(), s)));
  const int cap = capacity_of(c);
  return hip_status(moe::launch_permute_routed(
      idx, hist, counts, offsets, row_token, slot_row, region<int32_t>(ws, L, R_PERM_FLAGS),
      region<int32_t>(ws, L, R_GEN), gen_copy, T, E, k, cap < T ? cap : T, s));
}

// GEMM 1. `a` is x_perm (row_token == nullptr) or the token matrix x read through
// row_token (the permute gather fused into the operand loads).
moe_status do_up(const moe_config* c, const void* a, const int32_t* row_token,
                 const int32_t* offsets, const void* w_gate, const void* w_up, void* h,
                 hipStream_t s) {
  const int swiglu = c->activation == MOE_ACT_SWIGLU;
  const int epi = swiglu ? moe::EPI_SWIGLU : moe::EPI_GELU;
  const int rows = c->tokens * c->top_k;
  const int a_rows = row_token != nullptr ? c->tokens : rows;
  if (c->weight_layout & MOE_WEIGHTS_PACKED)
    return hip_status(moe::launch_gemm_bf16_packed(
        epi, (const moe::bf16_t*)a, row_token, a_rows, offsets,
        (const moe::bf16_t*)(swiglu ? w_gate : w_up), (const moe::bf16_t*)w_up,
        (moe::bf16_t*)h, nullptr, c->experts, c->hidden, c->inter, rows, s));
  if (c->dtype == MOE_DTYPE_BF16)
    return hip_status(moe::launch_gemm_bf16(
        epi, (const moe::bf16_t*)a, row_token, a_rows, offsets,
        (const moe::bf16_t*)(swiglu ? w_gate : w_up), (const moe::bf16_t*)w_up,
        (moe::bf16_t*)h, nullptr, nullptr, nullptr, c->experts, c->hidden, c->inter, rows, s));
  return hip_status(moe::launch_gemm_f32(epi, (const float*)a, row_token, a_rows, offsets,
                                         (const float*)(swiglu ? w_gate : w_up),
                                         (const float*)w_up, (float*)h, c->experts, c->hidden,
                                         c->inter, rows, s));
}

// GEMM 2. `partial` (bf16 only, may be null) is the split-K tail's scratch.
moe_status do_down(const moe_config* c, const void* h, const int32_t* offsets,
                   const void* w_down, void* y, float* partial, hipStream_t s) {
  const int rows = c->tokens * c->top_k;
  if (c->weight_layout & MOE_WEIGHTS_PACKED)
    return hip_status(moe::launch_gemm_bf16_packed(
        moe::EPI_NONE, (const moe::bf16_t*)h, nullptr, rows, offsets,
        (const moe::bf16_t*)w_down, nullptr, (moe::bf16_t*)y, partial, c->experts, c->inter,
        c->hidden, rows, s));
  if (c->dtype == MOE_DTYPE_BF16)
    return hip_status(moe::launch_gemm_bf16(moe::EPI_NONE, (const moe::bf16_t*)h, nullptr, rows,
                                            offsets, (const moe::bf16_t*)w_down, nullptr,
                                            (moe::bf16_t*)y, partial, nullptr, nullptr,
                                            c->experts, c->inter, c->hidden, rows, s));
  return hip_status(moe::launch_gemm_f32(moe::EPI_NONE, (const float*)h, nullptr, rows, offsets,
                                         (const float*)w_down, nullptr, (float*)y, c->experts,
                                         c->inter, c->hidden, rows, s));
}

moe_status do_combine(const moe_config* c, const void* y, const int32_t* slot_row,
                      const float* w, void* out, hipStream_t s) {
  return hip_status(moe::launch_combine(c->dtype == MOE_DTYPE_BF16, y, slot_row, w, out,
                                        c->tokens, c->hidden, c->top_k, s));
}

}  // namespace

extern "C" {

moe_status moe_workspace_size(const moe_config* cfg, size_t* bytes) {
  MOE_TRY(check_cfg(cfg));
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  *bytes = layout_of(cfg).total;
  return MOE_OK;
}

moe_status moe_capacity(const moe_config* cfg, int32_t* capacity) {
  MOE_TRY(check_cfg(cfg));
  if (capacity == nullptr) return MOE_ERR_INVALID_ARG;
  *capacity = capacity_of(cfg);
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* gate_bias, float* logits, int32_t* topk_idx, float* topk_w,
                     void* ws, size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->tokens == 0) return MOE_OK;   // empty batch: nothing to read or write
  if (x != nullptr) {
    MOE_TRY(need(x, 16));
    MOE_TRY(need(w_router, cfg->dtype == MOE_DTYPE_BF16 ? 16 : 4));
    if (gate_bias != nullptr) MOE_TRY(need(gate_bias, 4));
  }
  MOE_TRY(need(logits, 4));
  MOE_TRY(need(topk_idx, 4));
  MOE_TRY(need(topk_w, 4));
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  return do_route(cfg, x, w_router, gate_bias, logits, topk_idx, topk_w, ws,
                  (hipStream_t)stream);
}

moe_status moe_permute(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                       void* x_perm, int32_t* expert_counts, int32_t* expert_offsets,
                       int32_t* row_token, int32_t* slot_row, void* ws, size_t ws_bytes,
                       moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->tokens == 0) return MOE_OK;   // empty batch: nothing to read or write
  if (x_perm != nullptr) {   // NULL: row maps only
    MOE_TRY(need(x, 16));
    MOE_TRY(need(x_perm, 16));
  }
  MOE_TRY(need(topk_idx, 4));
  MOE_TRY(need(expert_counts, 4));
  MOE_TRY(need(expert_offsets, 4));
  MOE_TRY(need(row_token, 4));
  MOE_TRY(need(slot_row, 4));
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  return do_permute(cfg, x, topk_idx, x_perm, expert_counts, expert_offsets, row_token, slot_row,
                    ws, (hipStream_t)stream);
}

moe_status moe_route_permute(const moe_config* cfg, const void* x, const void* w_router,
                             const float* gate_bias, float* logits, int32_t* topk_idx,
                             float* topk_w, int32_t* expert_counts, int32_t* expert_offsets,
                             int32_t* row_token, int32_t* slot_row, void* ws, size_t ws_bytes,
                             moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->tokens == 0) return MOE_OK;   // empty batch: nothing to read or write
  if (x != nullptr) {
    MOE_TRY(need(x, 16));
    MOE_TRY(need(w_router, cfg->dtype == MOE_DTYPE_BF16 ? 16 : 4));
    if (gate_bias != nullptr) MOE_TRY(need(gate_bias, 4));
  }
  MOE_TRY(need(logits, 4));
  MOE_TRY(need(topk_idx, 4));
  MOE_TRY(need(topk_w, 4));
  MOE_TRY(need(expert_counts, 4));
  MOE_TRY(need(expert_offsets, 4));
  MOE_TRY(need(row_token, 4));
  MOE_TRY(need(slot_row, 4));
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  return do_route_permute(cfg, x, w_router, gate_bias, logits, topk_idx, topk_w, expert_counts,
                          expert_offsets, row_token, slot_row, ws, (hipStream_t)stream);
}

moe_status moe_permute_noalloc(const moe_config* cfg, const void* x, const int32_t* topk_idx,
                               void* x_perm, int32_t* expert_counts, int32_t* expert_offsets,
                               int32_t* row_token, int32_t* slot_row, int32_t* flags,
                               moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->tokens == 0) return MOE_OK;   // empty batch: nothing to read or write
  if (moe::permute_noalloc_words(cfg->tokens, cfg->experts) * 4 > MOE_NOALLOC_SCRATCH_BYTES)
    return MOE_ERR_WORKSPACE;            // beyond the library's fixed scratch
  if (x_perm != nullptr) {   // NULL: row maps only
    MOE_TRY(need(x, 16));
    MOE_TRY(need(x_perm, 16));
  }
  MOE_TRY(need(topk_idx, 4));
  MOE_TRY(need(expert_counts, 4));
  MOE_TRY(need(expert_offsets, 4));
  MOE_TRY(need(row_token, 4));
  MOE_TRY(need(slot_row, 4));
  if (flags != nullptr) MOE_TRY(need(flags, 4));
  const int cap = capacity_of(cfg);
  return hip_status(moe::launch_permute_noalloc(
      x, (int)esize(cfg), topk_idx, x_perm, expert_counts, expert_offsets, row_token, slot_row,
      flags, cfg->tokens, cfg->hidden, cfg->experts, cfg->top_k,
      cap < cfg->tokens ? cap : cfg->tokens, (hipStream_t)stream));
}

moe_status moe_expert_up(const moe_config* cfg, const void* x_perm,
                         const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                         void* h, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->tokens == 0) return MOE_OK;   // empty batch: nothing to read or write
  MOE_TRY(need(x_perm, 16));
  MOE_TRY(need(expert_offsets, 4));
  if (cfg->activation == MOE_ACT_SWIGLU) MOE_TRY(need(w_gate, 16));
  MOE_TRY(need(w_up, 16));
  MOE_TRY(need(h, 16));
  return do_up(cfg, x_perm, nullptr, expert_offsets, w_gate, w_up, h, (hipStream_t)stream);
}

moe_status moe_expert_up_rows(const moe_config* cfg, const void* x, const int32_t* row_token,
                              const int32_t* expert_offsets, const void* w_gate,
                              const void* w_up, void* h, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->tokens == 0) return MOE_OK;   // empty batch: nothing to read or write
  MOE_TRY(need(x, 16));
  MOE_TRY(need(row_token, 4));
  MOE_TRY(need(expert_offsets, 4));
  if (cfg->activation == MOE_ACT_SWIGLU) MOE_TRY(need(w_gate, 16));
  MOE_TRY(need(w_up, 16));
  MOE_TRY(need(h, 16));
  return do_up(cfg, x, row_token, expert_offsets, w_gate, w_up, h, (hipStream_t)stream);
}

moe_status moe_expert_down(const moe_config* cfg, const void* h, const int32_t* expert_offsets,
                           const void* w_down, void* y_perm, void* ws, size_t ws_bytes,
                           moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->tokens == 0) return MOE_OK;   // empty batch: nothing to read or write
  MOE_TRY(need(h, 16));
  MOE_TRY(need(expert_offsets, 4));
  MOE_TRY(need(w_down, 16));
  MOE_TRY(need(y_perm, 16));
  float* partial = nullptr;
  if (ws != nullptr) {
    MOE_TRY(check_ws(cfg, ws, ws_bytes));
    partial = region<float>(ws, layout_of(cfg), R_SPLIT);
  }
  return do_down(cfg, h, expert_offsets, w_down, y_perm, partial, (hipStream_t)stream);
}

moe_status moe_grouped_ffn(const moe_config* cfg, const void* x_perm,
                           const int32_t* expert_offsets, const void* w_gate, const void* w_up,
                           const void* w_down, void* y_perm, void* ws, size_t ws_bytes,
                           moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->tokens == 0) return MOE_OK;   // empty batch: nothing to read or write
  MOE_TRY(need(x_perm, 16));
  MOE_TRY(need(expert_offsets, 4));
  if (cfg->activation == MOE_ACT_SWIGLU) MOE_TRY(need(w_gate, 16));
  MOE_TRY(need(w_up, 16));
  MOE_TRY(need(w_down, 16));
  MOE_TRY(need(y_perm, 16));
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  const Layout L = layout_of(cfg);
  void* h = region<void>(ws, L, R_H);
  const hipStream_t s = (hipStream_t)stream;
  MOE_TRY(do_up(cfg, x_perm, nullptr, expert_offsets, w_gate, w_up, h, s));
  return do_down(cfg, h, expert_offsets, w_down, y_perm, region<float>(ws, L, R_SPLIT), s);
}

size_t moe_packed_weight_bytes(const moe_config* cfg, int32_t which) {
  if (cfg == nullptr || check_cfg(cfg) != MOE_OK || cfg->dtype != MOE_DTYPE_BF16) return 0;
  if (which == MOE_WEIGHT_ROUTER)
    return (size_t)moe::route_padded_experts(cfg->experts) * cfg->hidden * 2;
  if (which == MOE_WEIGHT_GATE && cfg->activation != MOE_ACT_SWIGLU) return 0;
  if (which == MOE_WEIGHT_GATE || which == MOE_WEIGHT_UP || which == MOE_WEIGHT_DOWN)
    return (size_t)cfg->experts * cfg->hidden * cfg->inter * 2;
  return 0;
}

moe_status moe_pack_expert_weight(const moe_config* cfg, int32_t which, const void* w,
                                  void* packed, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->dtype != MOE_DTYPE_BF16) return MOE_ERR_UNSUPPORTED;
  if (which == MOE_WEIGHT_ROUTER) {
    MOE_TRY(need(w, 2));
    MOE_TRY(need(packed, 16));
    const size_t wbytes = (size_t)cfg->hidden * cfg->experts * 2;
    const size_t pbytes = moe_packed_weight_bytes(cfg, which);
    const char* wb = (const char*)w;
    const char* pb = (const char*)packed;
    if (pb < wb + wbytes && wb < pb + pbytes) return MOE_ERR_INVALID_ARG;   // no overlap
    return hip_status(moe::launch_router_pack((const moe::bf16_t*)w, (moe::bf16_t*)packed,
                                              cfg->hidden, cfg->experts, (hipStream_t)stream));
  }
  int K, N;
  if (which == MOE_WEIGHT_GATE || which == MOE_WEIGHT_UP) {
    K = cfg->hidden;
    N = cfg->inter;
  } else if (which == MOE_WEIGHT_DOWN) {
    K = cfg->inter;
    N = cfg->hidden;
  } else {
    return MOE_ERR_INVALID_ARG;
  }
  if (which == MOE_WEIGHT_GATE && cfg->activation != MOE_ACT_SWIGLU) return MOE_ERR_INVALID_ARG;
  MOE_TRY(need(w, 16));
  MOE_TRY(need(packed, 16));
  const size_t bytes = (size_t)cfg->experts * K * N * 2;
  const char* wb = (const char*)w;
  const char* pb = (const char*)packed;
  if (pb < wb + bytes && wb < pb + bytes) return MOE_ERR_INVALID_ARG;   // must not overlap
  return hip_status(moe::launch_pack_weight_bf16((const moe::bf16_t*)w, (moe::bf16_t*)packed,
                                                 cfg->experts, K, N, (hipStream_t)stream));
}

moe_status moe_combine(const moe_config* cfg, const void* y_perm, const int32_t* slot_row,
                       const float* topk_w, void* out, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->tokens == 0) return MOE_OK;   // empty batch: nothing to read or write
  MOE_TRY(need(y_perm, 16));
  MOE_TRY(need(slot_row, 4));
  MOE_TRY(need(topk_w, 4));
  MOE_TRY(need(out, 16));
  return do_combine(cfg, y_perm, slot_row, topk_w, out, (hipStream_t)stream);
}

moe_status moe_forward(const moe_config* cfg, const void* x, const void* w_router,
                       const float* gate_bias, const void* w_gate, const void* w_up,
                       const void* w_down, void* out, void* ws, size_t ws_bytes,
                       moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  if (cfg->tokens == 0) return MOE_OK;   // empty batch: nothing to read or write
  MOE_TRY(need(x, 16));
  MOE_TRY(need(w_router, cfg->dtype == MOE_DTYPE_BF16 ? 16 : 4));
  if (gate_bias != nullptr) MOE_TRY(need(gate_bias, 4));
  if (cfg->activation == MOE_ACT_SWIGLU) MOE_TRY(need(w_gate, 16));
  MOE_TRY(need(w_up, 16));
  MOE_TRY(need(w_down, 16));
  MOE_TRY(need(out, 16));
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  const Layout L = layout_of(cfg);
  const hipStream_t s = (hipStream_t)stream;
  float* logits = region<float>(ws, L, R_LOGITS);
  int32_t* idx = region<int32_t>(ws, L, R_TOPK_IDX);
  float* w = region<float>(ws, L, R_TOPK_W);
  int32_t* counts = region<int32_t>(ws, L, R_COUNTS);
  int32_t* offsets = region<int32_t>(ws, L, R_OFFSETS);
  int32_t* slot_row = region<int32_t>(ws, L, R_SLOT_ROW);
  int32_t* row_token = region<int32_t>(ws, L, R_ROW_TOKEN);
  void* h = region<void>(ws, L, R_H);
  void* y = region<void>(ws, L, R_Y_PERM);
  // the permutation's row maps only: GEMM 1 gathers the token rows itself
  MOE_TRY(do_route_permute(cfg, x, w_router, gate_bias, logits, idx, w, counts, offsets,
                           row_token, slot_row, ws, s));
  MOE_TRY(do_up(cfg, x, row_token, offsets, w_gate, w_up, h, s));
  MOE_TRY(do_down(cfg, h, offsets, w_down, y, region<float>(ws, L, R_SPLIT), s));
  return do_combine(cfg, y, slot_row, w, out, s);
}

moe_status moe_forward_train(const moe_config* cfg, const void* x, const void* w_router,
                             const float* gate_bias, const void* w_gate, const void* w_up,
                             const void* w_down, void* out, void* ws, size_t ws_bytes,
                             void* bws, size_t bws_bytes, moe_stream_t stream) {
  MOE_TRY(check_backward_cfg(cfg));
  if (cfg->tokens == 0) return MOE_OK;   // empty batch: nothing to read or write
  MOE_TRY(need(x, 16));
  MOE_TRY(need(w_router, 16));
  if (gate_bias != nullptr) MOE_TRY(need(gate_bias, 4));
  if (cfg->activation == MOE_ACT_SWIGLU) MOE_TRY(need(w_gate, 16));
  MOE_TRY(need(w_up, 16));
  MOE_TRY(need(w_down, 16));
  MOE_TRY(need(out, 16));
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  if (bws == nullptr || !aligned(bws, 16)) return MOE_ERR_INVALID_ARG;
  if (bws_bytes < blayout_of(cfg).total) return MOE_ERR_WORKSPACE;
  const Layout L = layout_of(cfg);
  const BLayout B = blayout_of(cfg);
  const hipStream_t s = (hipStream_t)stream;
  float* logits = region<float>(ws, L, R_LOGITS);
  int32_t* idx = region<int32_t>(ws, L, R_TOPK_IDX);
  float* w = region<float>(ws, L, R_TOPK_W);
  int32_t* counts = region<int32_t>(ws, L, R_COUNTS);
  int32_t* offsets = region<int32_t>(ws, L, R_OFFSETS);
  int32_t* slot_row = region<int32_t>(ws, L, R_SLOT_ROW);
  int32_t* row_token = region<int32_t>(ws, L, R_ROW_TOKEN);
  moe::bf16_t* h = region<moe::bf16_t>(ws, L, R_H);
  void* y = region<void>(ws, L, R_Y_PERM);
  moe::bf16_t* gu = bregion<moe::bf16_t>(bws, B, B_GU);
  const int T = cfg->tokens, H = cfg->hidden, I = cfg->inter, E = cfg->experts;
  const int rows = T * cfg->top_k;
  MOE_TRY(do_route_permute(cfg, x, w_router, gate_bias, logits, idx, w, counts, offsets,
                           row_token, slot_row, ws, s, bregion<int32_t>(bws, B, B_GEN)));
  // GEMM 1 keeping the pre-activations for the backward: [g | u] (GELU: a) into bws, h as usual
  if (cfg->activation == MOE_ACT_SWIGLU)
    MOE_TRY(hip_status(moe::launch_gemm_bf16(
        moe::EPI_GU, (const moe::bf16_t*)x, row_token, T, offsets, (const moe::bf16_t*)w_gate,
        (const moe::bf16_t*)w_up, gu, nullptr, nullptr, h, E, H, I, rows, s)));
  else
    MOE_TRY(hip_status(moe::launch_gemm_bf16(
        moe::EPI_AH, (const moe::bf16_t*)x, row_token, T, offsets, (const moe::bf16_t*)w_up,
        nullptr, gu, nullptr, nullptr, h, E, H, I, rows, s)));
  MOE_TRY(do_down(cfg, h, offsets, w_down, y, region<float>(ws, L, R_SPLIT), s));
  return do_combine(cfg, y, slot_row, w, out, s);
}

moe_status moe_backward_workspace_size(const moe_config* cfg, size_t* bytes) {
  MOE_TRY(check_backward_cfg(cfg));
  if (bytes == nullptr) return MOE_ERR_INVALID_ARG;
  *bytes = blayout_of(cfg).total;
  return MOE_OK;
}

moe_status moe_backward(const moe_config* cfg, const void* x, const void* w_router,
                        const void* w_gate, const void* w_up, const void* w_down,
                        const void* dout, void* dx, float* dw_router, float* dgate_bias,
                        void* dw_gate, void* dw_up, void* dw_down, void* ws, size_t ws_bytes,
                        void* bws, size_t bws_bytes, int32_t saved, moe_stream_t stream) {
  MOE_TRY(check_backward_cfg(cfg));
  if (cfg->tokens == 0) return MOE_OK;   // empty batch: nothing to read or write
  const bool swiglu = cfg->activation == MOE_ACT_SWIGLU;
  MOE_TRY(need(x, 16));
  MOE_TRY(need(w_router, 16));
  if (swiglu) MOE_TRY(need(w_gate, 16));
  MOE_TRY(need(w_up, 16));
  MOE_TRY(need(w_down, 16));
  MOE_TRY(need(dout, 16));
  MOE_TRY(need(dx, 16));
  MOE_TRY(need(dw_router, 4));
  if (dgate_bias != nullptr) MOE_TRY(need(dgate_bias, 4));
  if (swiglu) MOE_TRY(need(dw_gate, 16));
  MOE_TRY(need(dw_up, 16));
  MOE_TRY(need(dw_down, 16));
  MOE_TRY(check_ws(cfg, ws, ws_bytes));
  if (bws == nullptr || !aligned(bws, 16)) return MOE_ERR_INVALID_ARG;
  if (bws_bytes < blayout_of(cfg).total) return MOE_ERR_WORKSPACE;
  using moe::bf16_t;
  const Layout L = layout_of(cfg);
  const BLayout B = blayout_of(cfg);
  const hipStream_t s = (hipStream_t)stream;
  const int T = cfg->tokens, H = cfg->hidden, I = cfg->inter, E = cfg->experts,
            k = cfg->top_k;
  const int P = moe::bwd_padded_rows(T, k, E);
  // the forward's intermediates
  const float* logits = region<float>(ws, L, R_LOGITS);
  const int32_t* idx = region<int32_t>(ws, L, R_TOPK_IDX);
  const float* w = region<float>(ws, L, R_TOPK_W);
  const int32_t* offsets = region<int32_t>(ws, L, R_OFFSETS);
  const int32_t* slot_row = region<int32_t>(ws, L, R_SLOT_ROW);
  const int32_t* row_token = region<int32_t>(ws, L, R_ROW_TOKEN);
  const bf16_t* y = region<bf16_t>(ws, L, R_Y_PERM);
  // the backward's own
  int32_t* poff = bregion<int32_t>(bws, B, B_POFF);
  int32_t* prow = bregion<int32_t>(bws, B, B_PROW);
  bf16_t* xP = bregion<bf16_t>(bws, B, B_XP);
  bf16_t* gu = bregion<bf16_t>(bws, B, B_GU);
  bf16_t* hP = bregion<bf16_t>(bws, B, B_H);
  bf16_t* dyP = bregion<bf16_t>(bws, B, B_DY);
  bf16_t* dgu = bregion<bf16_t>(bws, B, B_DGU);
  bf16_t* dxP = bregion<bf16_t>(bws, B, B_DXP);
  float* dL = bregion<float>(bws, B, B_DL);
  float* dwj = bregion<float>(bws, B, B_DW);
  float* split = bregion<float>(bws, B, B_SPLIT);
  const bf16_t* wg = (const bf16_t*)w_gate;
  const bf16_t* wu = (const bf16_t*)w_up;
  const bf16_t* wd = (const bf16_t*)w_down;

  // padded row maps and the token rows in padded expert-major order
  // (with saved pre-activations, also whether they belong to the latest permutation of ws)
  int32_t* gen = region<int32_t>(ws, L, R_GEN);
  MOE_TRY(hip_status(moe::launch_bwd_prepare((const bf16_t*)x, offsets, row_token, poff, prow,
                                             xP, gen, saved ? bregion<int32_t>(bws, B, B_GEN)
                                                            : nullptr,
                                             gen + 1, T, H, E, k, s)));
  // the up-projection's pre-activations: kept by moe_forward_train (compact rows, in bws), or
  // recomputed here in the padded row space together with h (GELU: a and h)
  if (saved) {   // h of the forward (ws), moved into the padded rows for dW_down
    MOE_TRY(hip_status(moe::launch_bwd_pad_copy(region<bf16_t>(ws, L, R_H), hP, offsets, poff, T,
                                                k, E, I / 8, s)));
  } else {
    if (swiglu)
      MOE_TRY(hip_status(moe::launch_gemm_bf16(moe::EPI_GU, xP, nullptr, P, poff, wg, wu, gu,
                                               nullptr, nullptr, hP, E, H, I, P, s)));
    else
      MOE_TRY(hip_status(moe::launch_gemm_bf16(moe::EPI_AH, xP, nullptr, P, poff, wu, nullptr,
                                               gu, nullptr, nullptr, hP, E, H, I, P, s)));
  }
  // combine backward: dy (padded, zero pads) and the gate-weight gradients
  MOE_TRY(hip_status(moe::launch_bwd_combine((const bf16_t*)dout, y, slot_row, idx, w, offsets,
                                             poff, dyP, dwj, T, H, E, k, s)));
  // the auxiliary load-balancing loss (its value into ws, its per-expert p-derivative for
  // the router backward), from the forward's logits and pre-capacity counts
  double* aux_g = nullptr;
  if (cfg->aux_loss_coeff > 0) {
    aux_g = bregion<double>(bws, B, B_AUXG);
    MOE_TRY(hip_status(moe::launch_bwd_aux_loss(logits, region<int32_t>(ws, L, R_COUNTS),
                                                bregion<double>(bws, B, B_AUXP), aux_g,
                                                region<double>(ws, L, R_AUX_LOSS), T, E,
                                                cfg->aux_loss_coeff, s)));
  }
  MOE_TRY(hip_status(moe::launch_bwd_router(logits, idx, dwj, aux_g, dL, T, E, k,
                                            cfg->renormalize != 0, s)));
  // dh = dy Wd^T with the activation's backward fused: [dg | du] (GELU: da). Wd[e] [I][H]
  // is Wd^T with K contiguous, read as is (transposed-weight mode).
  // (saved pre-activations are read through the compact row map)
  MOE_TRY(hip_status(moe::launch_gemm_bf16_bt(swiglu ? moe::EPI_SWIGLU_BWD : moe::EPI_GELU_BWD,
                                              dyP, poff, wd, nullptr, dgu, nullptr, gu,
                                              saved ? offsets : nullptr, E, H, I, P, s)));
  // dx rows = [dg | du] [Wg^T; Wu^T] (GELU: da Wu^T): one K = 2I product reading Wg[e] and
  // Wu[e] ([H][I] each, K contiguous) as the two K halves of the transposed weight
  MOE_TRY(hip_status(moe::launch_gemm_bf16_bt(moe::EPI_NONE, dgu, poff, swiglu ? wg : wu,
                                              swiglu ? wu : nullptr, dxP, split, nullptr,
                                              nullptr, E, swiglu ? 2 * I : I, H, P, s)));
  MOE_TRY(hip_status(moe::launch_bwd_dx(dxP, (const bf16_t*)w_router, dL, slot_row, idx,
                                        offsets, poff, (bf16_t*)dx, T, H, E, k, s)));
  MOE_TRY(hip_status(moe::launch_bwd_wrouter((const bf16_t*)x, dL, bregion<float>(bws, B, B_WRPART),
                                             bregion<float>(bws, B, B_BPART), dw_router,
                                             dgate_bias, T, H, E, s)));
  // weight gradients over each expert's padded rows. dy and the x rows reduce over rows as
  // a weight reduces over k, so they are packed once (the rows up to a multiple of 16 that
  // covers every expert's range) and loaded straight into registers; h and [dg | du] go
  // through LDS. dW_gate and dW_up are computed as dg^T x and du^T x and stored transposed.
  const int kpack = P / 16 * 16;
  bf16_t* xPk = bregion<bf16_t>(bws, B, B_XPK);
  bf16_t* dyPk = bregion<bf16_t>(bws, B, B_DYPK);
  MOE_TRY(hip_status(moe::launch_pack_weight_bf16(dyP, dyPk, 1, kpack, H, s)));
  MOE_TRY(hip_status(moe::launch_pack_weight_bf16(xP, xPk, 1, kpack, H, s)));
  MOE_TRY(hip_status(moe::launch_wgrad_bf16_packed(hP, I, dyPk, kpack, poff, (bf16_t*)dw_down,
                                                   E, I, H, 0, s)));
  if (swiglu) {
    MOE_TRY(hip_status(moe::launch_wgrad_bf16_packed(dgu, 2 * I, xPk, kpack, poff,
                                                     (bf16_t*)dw_gate, E, I, H, 1, s)));
    return hip_status(moe::launch_wgrad_bf16_packed(dgu + I, 2 * I, xPk, kpack, poff,
                                                    (bf16_t*)dw_up, E, I, H, 1, s));
  }
  return hip_status(moe::launch_wgrad_bf16_packed(dgu, I, xPk, kpack, poff, (bf16_t*)dw_up, E, I,
                                                  H, 1, s));
}

moe_status moe_workspace_view(const moe_config* cfg, void* ws, int32_t which, void** dev_ptr,
                              size_t* bytes) {
  MOE_TRY(check_cfg(cfg));
  if (ws == nullptr || dev_ptr == nullptr) return MOE_ERR_INVALID_ARG;
  static const Region map[MOE_WS_NUM_VIEWS] = {R_LOGITS,   R_TOPK_IDX, R_TOPK_W,  R_COUNTS,
                                               R_OFFSETS,  R_SLOT_ROW, R_ROW_TOKEN, R_NUM,
                                               R_H,        R_Y_PERM,   R_AUX_LOSS};
  if (which < 0 || which >= MOE_WS_NUM_VIEWS || map[which] == R_NUM) return MOE_ERR_INVALID_ARG;
  const Layout L = layout_of(cfg);
  *dev_ptr = static_cast<char*>(ws) + L.off[map[which]];
  if (bytes != nullptr) *bytes = L.size[map[which]];
  return MOE_OK;
}

moe_status moe_read_device_status(const moe_config* cfg, void* ws, int32_t which,
                                  moe_stream_t stream, int32_t* flags) {
  MOE_TRY(check_cfg(cfg));
  if (ws == nullptr || flags == nullptr || which < 1 || which > 7) return MOE_ERR_INVALID_ARG;
  *flags = 0;
  if (cfg->tokens == 0) return MOE_OK;
  const Layout L = layout_of(cfg);
  const hipStream_t s = (hipStream_t)stream;
  std::vector<int32_t> host;
  int32_t acc = 0;
  for (int part = 1; part <= 4; part <<= 1) {
    if (!(which & part)) continue;
    // route: one word per 16 tokens; permute: one per count block; backward: word 1 of R_GEN
    const Region r = part == 1 ? R_ROUTE_FLAGS : part == 2 ? R_PERM_FLAGS : R_GEN;
    const size_t off = part == 4 ? 4 : 0, bytes = part == 4 ? 4 : L.size[r];
    host.assign(bytes / 4, 0);
    MOE_TRY(hip_status(hipMemcpyAsync(host.data(), region<char>(ws, L, r) + off, bytes,
                                      hipMemcpyDeviceToHost, s)));
    MOE_TRY(hip_status(hipStreamSynchronize(s)));
    for (int32_t v : host) acc |= v;
  }
  *flags = acc;
  return MOE_OK;
}

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

int32_t moe_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
