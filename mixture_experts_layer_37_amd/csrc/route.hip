// Router: gate GEMM, softmax, top-k and gate weights for each token.
//
// The gate is a softmax over x @ W_gate followed by a top-k choice of experts
// (intelliparadigm.com, "MoE模型高效推理：CANN算子库优化实践", section 2.1; gitcode.csdn.net,
// "ops-transformer 仓库 - MoE 算子优化实战", "核心代码解析": routing_module_ -> TopKRouting).
// The pages sort the scores with a hardware bitonic sort (hnwysp.cn/news/132341, section
// 2.1, VectorizedTopK), which is not stable; here each token keeps a sorted register list
// of its best experts, filled in ascending expert order with a strict comparison, so among
// equal logits the lower expert index wins and the result is deterministic.
//
// bf16 path: the gate GEMM runs on MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
// x is streamed from HBM exactly once; the router weight is first transposed into the
// workspace as WT[E_pad][H] so that both MFMA operands are 16-byte K-contiguous loads.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace moe {

// Total order used for selection: -0.0 == +0.0, NaN below -inf, otherwise the float order.
__device__ __forceinline__ int order_key(float f) {
  if (f != f) return INT_MIN + 1;
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) return 0;
  return (u & 0x80000000u) ? (int)(u ^ 0x7fffffffu) : (int)u;
}

// Top-k of one token's E logits (any address space) and its gate weights. Weights are
// evaluated in float64 and rounded once to float32. Returns true if a logit is not finite.
template <int KMAX>
__device__ bool topk_token(const float* L, int E, int k, int renorm, int32_t* idx_out,
                           float* w_out) {
  int key[KMAX];
  int id[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) { key[j] = INT_MIN; id[j] = 0; }
  bool has_nan = false, nonfinite = false;
  for (int e = 0; e < E; ++e) {
    const float v = L[e];
    has_nan |= (v != v);
    nonfinite |= !__builtin_isfinite(v);
    const int kc = order_key(v);
    if (kc > key[KMAX - 1]) {
#pragma unroll
      for (int j = KMAX - 1; j > 0; --j) {
        const bool up = kc > key[j - 1];
        const bool here = kc > key[j];
        const int nk = up ? key[j - 1] : (here ? kc : key[j]);
        const int ni = up ? id[j - 1] : (here ? e : id[j]);
        key[j] = nk;
        id[j] = ni;
      }
      if (kc > key[0]) { key[0] = kc; id[0] = e; }
    }
  }
  const double top = (double)L[id[0]];
  double ev[KMAX];
  double s = 0.0;
  if (renorm) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) { ev[j] = exp((double)L[id[j]] - top); s += ev[j]; }
  } else {
    for (int e = 0; e < E; ++e) s += exp((double)L[e] - top);
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) ev[j] = exp((double)L[id[j]] - top);
  }
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      idx_out[j] = id[j];
      w_out[j] = has_nan ? __builtin_nanf("") : (float)(ev[j] / s);
    }
  }
  return nonfinite;
}

int route_padded_experts(int E) {
  return E <= 16 ? 16 : E <= 32 ? 32 : E <= 64 ? 64 : E <= 128 ? 128 : 256;
}

// WT[e][h] = W[h][e] for e < E, 0 for E <= e < E_pad. One thread per (e, 8 consecutive h).
__global__ __launch_bounds__(256) void router_transpose_kernel(const bf16_t* __restrict__ w,
                                                               bf16_t* __restrict__ wt, int H,
                                                               int E, int EP) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  const int e = i % EP, hc = i / EP;
  if (hc * 8 >= H) return;
  uint32_t d[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t lo = 0, hi = 0;
    if (e < E) {
      lo = w[(size_t)(hc * 8 + 2 * q) * E + e];
      hi = w[(size_t)(hc * 8 + 2 * q + 1) * E + e];
    }
    d[q] = lo | (hi << 16);
  }
  *(uint4*)(wt + (size_t)e * H + hc * 8) = make_uint4(d[0], d[1], d[2], d[3]);
}

hipError_t launch_router_transpose(const bf16_t* w, bf16_t* wt, int H, int E, hipStream_t s) {
  const int EP = route_padded_experts(E);
  const long n = (long)EP * (H / 8);
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(router_transpose_kernel, dim3(blocks), dim3(256), 0, s, w, wt, H, E, EP);
  return hipGetLastError();
}

// Gate GEMM on MFMA + top-k. A block of 4 waves owns BT = 16*TG tokens; wave w sums over
// its quarter of H, the four partial [BT x 16*NBE] tiles are added in a fixed order through
// LDS, then threads 0..BT-1 each select the experts of one token.
template <int TG, int NBE, int KMAX>
__global__ __launch_bounds__(256) void route_mfma_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wt, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ flags, int T, int H, int E, int k, int renorm) {
  constexpr int BT = TG * 16, EP = NBE * 16, LDR = EP + 1;
  constexpr int U = (TG + NBE) >= 12 ? 1 : (12 / (TG + NBE) < 8 ? 12 / (TG + NBE) : 8);
  __shared__ float red[2][BT * LDR];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * BT;
  const int nchunk = H / 32;
  const int c0 = wave * nchunk / 4, c1 = (wave + 1) * nchunk / 4;

  f32x4 acc[TG][NBE];
#pragma unroll
  for (int g = 0; g < TG; ++g)
#pragma unroll
    for (int n = 0; n < NBE; ++n) acc[g][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bf16_t* xr[TG];
#pragma unroll
  for (int g = 0; g < TG; ++g) {
    int row = t0 + g * 16 + (lane & 15);
    row = row < T ? row : T - 1;
    xr[g] = x + (size_t)row * H + (lane >> 4) * 8;
  }
  const bf16_t* wr[NBE];
#pragma unroll
  for (int n = 0; n < NBE; ++n) wr[n] = wt + (size_t)(n * 16 + (lane & 15)) * H + (lane >> 4) * 8;

  int c = c0;
  for (; c + U <= c1; c += U) {
    bf16x8 a[U][TG], b[U][NBE];
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int g = 0; g < TG; ++g) a[u][g] = *(const bf16x8*)(xr[g] + (c + u) * 32);
#pragma unroll
      for (int n = 0; n < NBE; ++n) b[u][n] = *(const bf16x8*)(wr[n] + (c + u) * 32);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < TG; ++g)
#pragma unroll
        for (int n = 0; n < NBE; ++n)
          acc[g][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[u][g], b[u][n], acc[g][n], 0, 0, 0);
  }
  for (; c < c1; ++c) {
    bf16x8 a[TG], b[NBE];
#pragma unroll
    for (int g = 0; g < TG; ++g) a[g] = *(const bf16x8*)(xr[g] + c * 32);
#pragma unroll
    for (int n = 0; n < NBE; ++n) b[n] = *(const bf16x8*)(wr[n] + c * 32);
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
      for (int n = 0; n < NBE; ++n)
        acc[g][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[g], b[n], acc[g][n], 0, 0, 0);
  }

  // Fixed-order reduction of the four K-quarters: (w0 + w2) + (w1 + w3).
  // MFMA 16x16 output: lane holds column (expert) lane&15, rows 4*(lane>>4) + r.
  auto tile_at = [&](float* buf, int g, int n, int r) -> float& {
    return buf[(g * 16 + (lane >> 4) * 4 + r) * LDR + n * 16 + (lane & 15)];
  };
  if (wave >= 2) {
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
      for (int n = 0; n < NBE; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) tile_at(red[wave - 2], g, n, r) = acc[g][n][r];
  }
  __syncthreads();
  if (wave < 2) {
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
      for (int n = 0; n < NBE; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[g][n][r] += tile_at(red[wave], g, n, r);
  }
  __syncthreads();
  if (wave == 1) {
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
      for (int n = 0; n < NBE; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) tile_at(red[0], g, n, r) = acc[g][n][r];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int g = 0; g < TG; ++g)
#pragma unroll
      for (int n = 0; n < NBE; ++n) {
        const int e = n * 16 + (lane & 15);
        const float b = (bias != nullptr && e < E) ? bias[e] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float& slot = tile_at(red[0], g, n, r);
          slot = (acc[g][n][r] + slot) + b;
        }
      }
  }
  __syncthreads();

  const float* Ls = red[0];
  for (int i = threadIdx.x; i < BT * E; i += blockDim.x) {
    const int t = i / E, e = i - t * E;
    if (t0 + t < T) logits[(size_t)(t0 + t) * E + e] = Ls[t * LDR + e];
  }
  if (threadIdx.x < 64) {
    bool nf = false;
    const int t = t0 + threadIdx.x;
    if (threadIdx.x < BT && t < T)
      nf = topk_token<KMAX>(Ls + threadIdx.x * LDR, E, k, renorm, topk_idx + (size_t)t * k,
                            topk_w + (size_t)t * k);
    const unsigned long long m = __ballot(nf);
    const int ngroups = (T + kRouteFlagGroup - 1) / kRouteFlagGroup;
    if (threadIdx.x < TG && blockIdx.x * TG + threadIdx.x < ngroups)
      flags[blockIdx.x * TG + threadIdx.x] =
          ((m >> (16 * threadIdx.x)) & 0xffffull) ? 2 /* MOE_FLAG_NONFINITE_LOGIT */ : 0;
  }
}

template <int TG, int NBE>
static hipError_t launch_route_tg(const bf16_t* x, const bf16_t* wt, const float* bias,
                                  float* logits, int32_t* idx, float* w, int32_t* flags, int T,
                                  int H, int E, int k, int renorm, hipStream_t s) {
  const dim3 grid((T + TG * 16 - 1) / (TG * 16)), block(256);
#define MOE_ROUTE_LAUNCH(KM)                                                                  \
  hipLaunchKernelGGL((route_mfma_kernel<TG, NBE, KM>), grid, block, 0, s, x, wt, bias, logits, \
                     idx, w, flags, T, H, E, k, renorm)
  if (k <= 1) MOE_ROUTE_LAUNCH(1);
  else if (k <= 2) MOE_ROUTE_LAUNCH(2);
  else if (k <= 4) MOE_ROUTE_LAUNCH(4);
  else if (k <= 8) MOE_ROUTE_LAUNCH(8);
  else MOE_ROUTE_LAUNCH(16);
#undef MOE_ROUTE_LAUNCH
  return hipGetLastError();
}

hipError_t launch_route_bf16(const bf16_t* x, const bf16_t* wt, const float* bias, float* logits,
                             int32_t* idx, float* w, int32_t* flags, int T, int H, int E, int k,
                             int renorm, hipStream_t s) {
  switch (route_padded_experts(E)) {
    case 16: return launch_route_tg<1, 1>(x, wt, bias, logits, idx, w, flags, T, H, E, k, renorm, s);
    case 32: return launch_route_tg<1, 2>(x, wt, bias, logits, idx, w, flags, T, H, E, k, renorm, s);
    case 64: return launch_route_tg<2, 4>(x, wt, bias, logits, idx, w, flags, T, H, E, k, renorm, s);
    case 128: return launch_route_tg<4, 8>(x, wt, bias, logits, idx, w, flags, T, H, E, k, renorm, s);
    default: return launch_route_tg<2, 16>(x, wt, bias, logits, idx, w, flags, T, H, E, k, renorm, s);
  }
}

// fp32 gate GEMM on the vector ALUs: one thread per (token, expert), h in ascending order.
__global__ __launch_bounds__(256) void route_logits_f32_kernel(const float* __restrict__ x,
                                                               const float* __restrict__ w,
                                                               const float* __restrict__ bias,
                                                               float* __restrict__ logits,
                                                               int T, int H, int E) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long)T * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  const float* xr = x + (size_t)t * H;
  float acc = 0.f;
  for (int h = 0; h < H; ++h) acc = fmaf(xr[h], w[(size_t)h * E + e], acc);
  logits[i] = acc + (bias != nullptr ? bias[e] : 0.f);
}

hipError_t launch_route_logits_f32(const float* x, const float* w, const float* bias,
                                   float* logits, int T, int H, int E, hipStream_t s) {
  const long n = (long)T * E;
  hipLaunchKernelGGL(route_logits_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     s, x, w, bias, logits, T, H, E);
  return hipGetLastError();
}

// Top-k from logits already in memory: one thread per token, 64 tokens per block.
template <int KMAX>
__global__ __launch_bounds__(64) void route_topk_kernel(const float* __restrict__ logits,
                                                        int32_t* __restrict__ idx,
                                                        float* __restrict__ w,
                                                        int32_t* __restrict__ flags, int T,
                                                        int E, int k, int renorm) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  bool nf = false;
  if (t < T)
    nf = topk_token<KMAX>(logits + (size_t)t * E, E, k, renorm, idx + (size_t)t * k,
                          w + (size_t)t * k);
  const unsigned long long m = __ballot(nf);
  const int ngroups = (T + kRouteFlagGroup - 1) / kRouteFlagGroup;
  const int g = blockIdx.x * 4 + threadIdx.x;
  if (threadIdx.x < 4 && g < ngroups)
    flags[g] = ((m >> (16 * threadIdx.x)) & 0xffffull) ? 2 /* MOE_FLAG_NONFINITE_LOGIT */ : 0;
}

hipError_t launch_route_topk(const float* logits, int32_t* idx, float* w, int32_t* flags, int T,
                             int E, int k, int renorm, hipStream_t s) {
  const dim3 grid((T + 63) / 64), block(64);
#define MOE_TOPK_LAUNCH(KM) \
  hipLaunchKernelGGL((route_topk_kernel<KM>), grid, block, 0, s, logits, idx, w, flags, T, E, k, renorm)
  if (k <= 1) MOE_TOPK_LAUNCH(1);
  else if (k <= 2) MOE_TOPK_LAUNCH(2);
  else if (k <= 4) MOE_TOPK_LAUNCH(4);
  else if (k <= 8) MOE_TOPK_LAUNCH(8);
  else MOE_TOPK_LAUNCH(16);
#undef MOE_TOPK_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
