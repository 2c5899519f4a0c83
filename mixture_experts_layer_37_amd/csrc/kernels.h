// Internal launch wrappers of the MoE kernels (one translation unit per step). Each returns
// the HIP error of its launch(es); shapes are validated by the caller (moe_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace moe {

// ---- route (route.hip). renorm: renormalised weights; thr: threshold routing with `delta`
int route_padded_experts(int E);
// w_router [H][E] -> wt: MFMA operands [E_pad / 16][H / 32][64][8] (E_pad =
// route_padded_experts(E)), zeros past E; the general router (launch_route_bf16) reads wt
hipError_t launch_router_pack(const bf16_t* w_router, bf16_t* wt, int H, int E, hipStream_t s);
hipError_t launch_route_bf16(const bf16_t* x, const bf16_t* wt, const float* bias,
                             float* logits, int32_t* topk_idx, float* topk_w, int32_t* flags,
                             int T, int H, int E, int k, int renorm, int thr, double delta,
                             hipStream_t s);
bool route_lds_fits(int H, int E);
// Tokens per block of the streaming router, which is also the count block of the
// permutation it can count (cnt_hist / cnt_rank below).
constexpr int kRouteCountTokens = 32;
// the streaming router: w_router [H][E] as it is, or (w_router == nullptr) wt, the same
// weight in launch_router_pack's layout. cnt_hist (may be null: no count): the
// permutation's count step as well, per block of kRouteCountTokens tokens the per-expert
// assignment counts into cnt_hist [ceil(T / 32)][E], and each slot's rank among its block's
// assignments to its expert (token order; -1 for an empty slot) into cnt_rank [T][k]
hipError_t launch_route_bf16_lds(const bf16_t* x, const bf16_t* w_router, const bf16_t* wt,
                                 const float* bias, float* logits, int32_t* topk_idx,
                                 float* topk_w, int32_t* flags, int32_t* cnt_hist,
                                 int32_t* cnt_rank, int T, int H, int E, int k, int renorm,
                                 int thr, double delta, int cus, hipStream_t s);
int device_cus();
hipError_t launch_route_logits_f32(const float* x, const float* w_router, const float* bias,
                                   float* logits, int T, int H, int E, hipStream_t s);
hipError_t launch_route_topk(const float* logits, int32_t* topk_idx, float* topk_w,
                             int32_t* flags, int T, int E, int k, int renorm, int thr,
                             double delta, hipStream_t s);

// ---- permute (permute.hip)
int permute_count_blocks(int T);
// Batches of at most this many count blocks (65536 tokens) get the scan and their row maps
// from one launch after the count (permute_scan_rows_kernel), each block reading the whole
// histogram table.
constexpr int kMapsMaxBlocks = 64;
// gen (may be null): the workspace's permutation generation, advanced by one; gen_copy (may
// be null): receives the new value (a training forward's record of it); flag_out (may be
// null): the OR of the per-block flags
hipError_t launch_permute(const void* x, int elem_bytes, const int32_t* topk_idx, void* x_perm,
                          int32_t* counts, int32_t* offsets, int32_t* row_token,
                          int32_t* slot_row, int32_t* hist, int32_t* flags, int32_t* gen,
                          int32_t* gen_copy, int32_t* flag_out, int T, int H, int E, int k,
                          int cap, hipStream_t s);
// The row maps of the permutation whose count step the streaming router did
// (launch_route_bf16_lds with cnt_hist): one launch, permute_scan_rows_kernel over count
// blocks of kRouteCountTokens tokens. slot_row holds the router's ranks on entry and the
// rows on return; perm_flags (the count kernel's flag words, ceil(T / 1024) of them) are
// cleared, since the router's ids are valid by construction. At most kRoutedMaxBlocks
// count blocks.
constexpr int kRoutedMaxBlocks = 8192;
hipError_t launch_permute_routed(const int32_t* topk_idx, const int32_t* cnt_hist,
                                 int32_t* counts, int32_t* offsets, int32_t* row_token,
                                 int32_t* slot_row, int32_t* perm_flags, int32_t* gen,
                                 int32_t* gen_copy, int T, int E, int k, int cap,
                                 hipStream_t s);
// The same permutation with its scratch in a file-scope device array of kNoAllocScratchWords
// int32 words (no workspace, no allocation): permute_noalloc_words(T, E) words are used;
// more -> hipErrorInvalidValue, before any HIP call. flag_out (may be null) as above.
constexpr int kNoAllocScratchWords = 1 << 18;   // 1 MiB
size_t permute_noalloc_words(int T, int E);
hipError_t launch_permute_noalloc(const void* x, int elem_bytes, const int32_t* topk_idx,
                                  void* x_perm, int32_t* counts, int32_t* offsets,
                                  int32_t* row_token, int32_t* slot_row, int32_t* flag_out,
                                  int T, int H, int E, int k, int cap, hipStream_t s);

// ---- grouped expert GEMMs (gemm.hip)
// Epilogues: SWIGLU h = silu(g) u; GELU h = gelu(a); NONE the product itself; GU the gate
// and up pre-activations into a [rows, 2N] pair buffer and h into `c2`; AH a into c and
// gelu(a) into `c2`; SWIGLU_BWD / GELU_BWD the activation's backward from the product dh and
// the saved pre-activations in `aux` (SWIGLU_BWD writes the [dg | du] pair buffer).
enum Epilogue { EPI_SWIGLU = 0, EPI_GELU = 1, EPI_NONE = 2, EPI_GU = 3, EPI_SWIGLU_BWD = 4,
                EPI_GELU_BWD = 5, EPI_AH = 6 };
// A row r of the expert-major operand is a[r], or a[row_token[r]] when row_token is given
// (token rows gathered in place; indexes clamped into [0, a_rows)).
// `partial` (EPI_NONE only; may be null): float32 scratch of kSplitPartialBytes for the
// split-K tail; null runs every tile whole.
constexpr int kSplitMaxUnits = 256;   // K slices of one launch, at most
constexpr size_t kSplitPartialBytes = (size_t)kSplitMaxUnits * 256 * 256 * 4;
hipError_t launch_gemm_bf16(int epi, const bf16_t* a, const int32_t* row_token, int a_rows,
                            const int32_t* offsets, const bf16_t* w0, const bf16_t* w1,
                            bf16_t* c, float* partial, const bf16_t* aux, bf16_t* c2, int E,
                            int K, int N, int max_rows, hipStream_t s);
hipError_t launch_gemm_f32(int epi, const float* a, const int32_t* row_token, int a_rows,
                           const int32_t* offsets, const float* w0, const float* w1, float* c,
                           int E, int K, int N, int max_rows, hipStream_t s);

// As launch_gemm_bf16 with the weights given transposed: w0 (and w1) [E][N][Ks] with K
// contiguous; with w1, k < K/2 reads w0 and k >= K/2 reads w1 (Ks = K/2), else Ks = K.
// Single-matrix epilogues (NONE with the split-K tail, SWIGLU_BWD, GELU_BWD); A plain rows.
// aux_off (may be null): the aux rows are compact, row r of expert e at
// r - offsets[e] + aux_off[e] (pad rows: the expert's last row).
hipError_t launch_gemm_bf16_bt(int epi, const bf16_t* a, const int32_t* offsets,
                               const bf16_t* w0, const bf16_t* w1, bf16_t* c, float* partial,
                               const bf16_t* aux, const int32_t* aux_off, int E, int K, int N,
                               int max_rows, hipStream_t s);
// Packed weights: W [E][K][N] -> P of the same size, P[e][N/32][K/16][64][8] with lane l's
// 8 values of block (nb, ks) = W[e][16 ks + 8 (l >> 5) + 0..7][32 nb + (l & 31)].
hipError_t launch_pack_weight_bf16(const bf16_t* w, bf16_t* packed, int E, int K, int N,
                                   hipStream_t s);
// As launch_gemm_bf16 with packed weights (SWIGLU: p0 gate, p1 up; GELU, NONE: p0), for the
// forward epilogues only; bit-identical results.
hipError_t launch_gemm_bf16_packed(int epi, const bf16_t* a, const int32_t* row_token,
                                   int a_rows, const int32_t* offsets, const bf16_t* p0,
                                   const bf16_t* p1, bf16_t* c, float* partial, int E, int K,
                                   int N, int max_rows, hipStream_t s);
// Weight gradients C_e = A_e^T B_e over each expert's padded rows poff[e] .. poff[e+1]
// (multiples of 128): A [rows][lda] row-major, B packed over the whole padded row space
// (pack_weight_kernel's layout, E = 1, K = kpack rows, a multiple of 16 covering poff[E]);
// M, N multiples of 256; trans_out stores C^T ([E][N][M]).
hipError_t launch_wgrad_bf16_packed(const bf16_t* a, int lda, const bf16_t* pb, int kpack,
                                    const int32_t* poff, bf16_t* c, int E, int M, int N,
                                    int trans_out, hipStream_t s);

// ---- backward pass (backward.hip): padded row space, multiples of 128 rows per expert
int bwd_padded_rows(int T, int k, int E);
int bwd_wrouter_chunks(int T);
// gen / gen_saved (gen_saved may be null: no saved pre-activations): bflag = 4 (stale saved
// pre-activations) when they differ, else 0
hipError_t launch_bwd_prepare(const bf16_t* x, const int32_t* offsets, const int32_t* row_token,
                              int32_t* poff, int32_t* prow_token, bf16_t* xP,
                              const int32_t* gen, const int32_t* gen_saved, int32_t* bflag,
                              int T, int H, int E, int k, hipStream_t s);
// dst[r] = src[compact row of padded row r] for r < poff[E] (rows of `row_vecs` 16-byte
// vectors; pad rows repeat the expert's last kept row).
hipError_t launch_bwd_pad_copy(const bf16_t* src, bf16_t* dst, const int32_t* offsets,
                               const int32_t* poff, int T, int k, int E, int row_vecs,
                               hipStream_t s);
hipError_t launch_bwd_combine(const bf16_t* dout, const bf16_t* y, const int32_t* slot_row,
                              const int32_t* topk_idx, const float* topk_w,
                              const int32_t* offsets, const int32_t* poff, bf16_t* dyP,
                              float* dw, int T, int H, int E, int k, hipStream_t s);
// aux_g: per-expert derivative of the auxiliary loss with respect to p (or nullptr: none)
hipError_t launch_bwd_router(const float* logits, const int32_t* topk_idx, const float* dw,
                             const double* aux_g, float* dL, int T, int E, int k, int renorm,
                             hipStream_t s);
// Auxiliary load-balancing loss: part [bwd_aux_blocks(T) * E] float64 scratch; g [E] and
// loss [1] float64 out
int bwd_aux_blocks(int T);
hipError_t launch_bwd_aux_loss(const float* logits, const int32_t* counts, double* part,
                               double* g, double* loss, int T, int E, double coeff,
                               hipStream_t s);
hipError_t launch_bwd_dx(const bf16_t* dxP, const bf16_t* w_router, const float* dL,
                         const int32_t* slot_row, const int32_t* topk_idx,
                         const int32_t* offsets, const int32_t* poff, bf16_t* dx, int T, int H,
                         int E, int k, hipStream_t s);
hipError_t launch_bwd_wrouter(const bf16_t* x, const float* dL, float* part, float* bpart,
                              float* dwr, float* dbias, int T, int H, int E, hipStream_t s);

// ---- combine (combine.hip)
hipError_t launch_combine(int dtype_bf16, const void* y, const int32_t* slot_row,
                          const float* topk_w, void* out, int T, int H, int k, hipStream_t s);

}  // namespace moe
