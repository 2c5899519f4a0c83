// Internal launch wrappers of the MoE kernels (one translation unit per step). Each returns
// the HIP error of its launch(es); shapes are validated by the caller (moe_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace moe {

// ---- route (route.hip). renorm: renormalised weights; thr: threshold routing with `delta`
int route_padded_experts(int E);
hipError_t launch_router_transpose(const bf16_t* w_router, bf16_t* wt, int H, int E,
                                   hipStream_t s);
hipError_t launch_route_bf16(const bf16_t* x, const bf16_t* wt, const float* bias,
                             float* logits, int32_t* topk_idx, float* topk_w, int32_t* flags,
                             int T, int H, int E, int k, int renorm, int thr, double delta,
                             hipStream_t s);
bool route_lds_fits(int H, int E);
hipError_t launch_route_bf16_lds(const bf16_t* x, const bf16_t* w_router, const float* bias,
                                 float* logits, int32_t* topk_idx, float* topk_w, int32_t* flags,
                                 int T, int H, int E, int k, int renorm, int thr, double delta,
                                 int cus, hipStream_t s);
int device_cus();
hipError_t launch_route_logits_f32(const float* x, const float* w_router, const float* bias,
                                   float* logits, int T, int H, int E, hipStream_t s);
hipError_t launch_route_topk(const float* logits, int32_t* topk_idx, float* topk_w,
                             int32_t* flags, int T, int E, int k, int renorm, int thr,
                             double delta, hipStream_t s);

// ---- permute (permute.hip)
int permute_count_blocks(int T);
hipError_t launch_permute(const void* x, int elem_bytes, const int32_t* topk_idx, void* x_perm,
                          int32_t* counts, int32_t* offsets, int32_t* row_token,
                          int32_t* slot_row, int32_t* hist, int32_t* flags, int T, int H,
                          int E, int k, int cap, hipStream_t s);

// ---- grouped expert GEMMs (gemm.hip)
enum Epilogue { EPI_SWIGLU = 0, EPI_GELU = 1, EPI_NONE = 2 };
// A row r of the expert-major operand is a[r], or a[row_token[r]] when row_token is given
// (token rows gathered in place; indexes clamped into [0, a_rows)).
// `partial` (EPI_NONE only; may be null): float32 scratch of kSplitPartialBytes for the
// split-K tail; null runs every tile whole.
constexpr int kSplitMaxUnits = 256;   // K slices of one launch, at most
constexpr size_t kSplitPartialBytes = (size_t)kSplitMaxUnits * 256 * 256 * 4;
hipError_t launch_gemm_bf16(int epi, const bf16_t* a, const int32_t* row_token, int a_rows,
                            const int32_t* offsets, const bf16_t* w0, const bf16_t* w1,
                            bf16_t* c, float* partial, int E, int K, int N, int max_rows,
                            hipStream_t s);
hipError_t launch_gemm_f32(int epi, const float* a, const int32_t* row_token, int a_rows,
                           const int32_t* offsets, const float* w0, const float* w1, float* c,
                           int E, int K, int N, int max_rows, hipStream_t s);

// ---- combine (combine.hip)
hipError_t launch_combine(int dtype_bf16, const void* y, const int32_t* slot_row,
                          const float* topk_w, void* out, int T, int H, int k, hipStream_t s);

}  // namespace moe
