// Backward pass of the layer: the kernels around the grouped GEMMs.
//
// The pages run the backward on the selected experts only (gitcode.csdn.net,
// "ops-transformer 仓库 - MoE 算子优化实战", "MoE 算子核心原理": sparse computation runs
// forward and backward on the chosen experts); each step here is the chain rule of one
// forward step. The backward works in a padded row space: expert e owns rows
// [poff[e], poff[e+1]), its kept rows first, then zero-gradient pad rows up to a multiple of
// 128, so the weight-gradient GEMMs reduce over whole 64-row k-steps in pairs.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int kPadRows = 128;

// poff[E+1]: padded row offsets from the kept offsets (clamped to [0, max_rows]). With saved
// pre-activations (gen_saved != null), bflag records whether they were kept by the training
// forward of the workspace's latest permutation (0) or not (4: stale).
__global__ void bwd_pad_offsets_kernel(const int32_t* __restrict__ offsets,
                                       int32_t* __restrict__ poff, int E, int max_rows,
                                       const int32_t* __restrict__ gen,
                                       const int32_t* __restrict__ gen_saved,
                                       int32_t* __restrict__ bflag) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  bflag[0] = (gen_saved != nullptr && gen_saved[0] != gen[0]) ? 4 /* MOE_FLAG_STALE_SAVED */ : 0;
  int acc = 0, prev = min(max(offsets[0], 0), max_rows);
  poff[0] = 0;
  for (int e = 0; e < E; ++e) {
    const int nxt = min(max(offsets[e + 1], 0), max_rows);
    const int m = max(nxt - prev, 0);
    acc += (m + kPadRows - 1) / kPadRows * kPadRows;
    poff[e + 1] = acc;
    prev = max(nxt, prev);
  }
}

// Largest e with poff[e] <= r (poff non-decreasing, r < poff[E]).
__device__ __forceinline__ int find_padded_expert(const int32_t* poff, int E, int r) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (poff[mid] <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// One wave per padded row r < poff[E]: prow_token[r] = the token of kept row r of its
// expert (pad rows repeat the expert's last kept row), and xP[r] = x[prow_token[r]].
__global__ __launch_bounds__(256) void bwd_pad_rows_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ poff, const int32_t* __restrict__ row_token,
    int32_t* __restrict__ prow_token, uint4* __restrict__ xP, int E, int T, int nrows,
    int prows_max, int row_vecs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= prows_max || r >= poff[E]) return;
  const int e = find_padded_expert(poff, E, r);
  const int m = offsets[e + 1] - offsets[e];   // > 0: the expert owns padded rows
  const int src = min(max(offsets[e] + min(r - poff[e], m - 1), 0), nrows - 1);
  const int t = min(max(row_token[src], 0), T - 1);
  if (lane == 0) prow_token[r] = t;
  const uint4* s = x + (size_t)t * row_vecs;
  uint4* d = xP + (size_t)r * row_vecs;
  for (int c = lane; c < row_vecs; c += 64) d[c] = s[c];
}

// One wave per padded row r < poff[E]: dst[r] = src[the compact row of r] (pad rows repeat
// the expert's last kept row).
__global__ __launch_bounds__(256) void bwd_pad_copy_kernel(
    const uint4* __restrict__ src, uint4* __restrict__ dst, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ poff, int E, int nrows, int prows_max, int row_vecs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + wave;
  if (r >= prows_max || r >= poff[E]) return;
  const int e = find_padded_expert(poff, E, r);
  const int m = offsets[e + 1] - offsets[e];
  const int c = min(max(offsets[e] + min(r - poff[e], m - 1), 0), nrows - 1);
  const uint4* s = src + (size_t)c * row_vecs;
  uint4* d = dst + (size_t)r * row_vecs;
  for (int i = lane; i < row_vecs; i += 64) d[i] = s[i];
}

// Combine backward, one wave per token: for each kept slot j (row r of expert e),
// dyP[padded r] = w_j dout[t] (bf16) and dw[t,j] = <dout[t], y[r]> (float32, lane partial
// sums in column order, then a fixed butterfly); dw = 0 for slots not kept.
template <int KMAX>
__global__ __launch_bounds__(256) void bwd_combine_kernel(
    const bf16_t* __restrict__ dout, const bf16_t* __restrict__ y,
    const int32_t* __restrict__ slot_row, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ topk_w, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ poff, bf16_t* __restrict__ dyP, float* __restrict__ dw, int T,
    int H, int E, int k, int nrows, int prows) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int nvec = H / 8;
  const bf16_t* drow = dout + (size_t)t * H;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j >= k) break;
    const int r = slot_row[(size_t)t * k + j];
    const int e = topk_idx[(size_t)t * k + j];
    if (r < 0 || r >= nrows || e < 0 || e >= E) {
      if (lane == 0) dw[(size_t)t * k + j] = 0.f;
      continue;
    }
    const float wj = topk_w[(size_t)t * k + j];
    const int pr = r - offsets[e] + poff[e];
    if (pr < 0 || pr >= prows) {   // inconsistent maps: never write outside dyP
      if (lane == 0) dw[(size_t)t * k + j] = 0.f;
      continue;
    }
    const bf16_t* yrow = y + (size_t)r * H;
    bf16_t* orow = dyP + (size_t)pr * H;
    float part = 0.f;
    for (int c = lane; c < nvec; c += 64) {
      const uint4 dv = *(const uint4*)(drow + c * 8);
      const uint4 yv = *(const uint4*)(yrow + c * 8);
      const uint32_t dw32[4] = {dv.x, dv.y, dv.z, dv.w};
      const uint32_t yw32[4] = {yv.x, yv.y, yv.z, yv.w};
      float o[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float d0 = bf16_to_f32(dw32[q] & 0xffffu), d1 = bf16_to_f32(dw32[q] >> 16);
        part = fmaf(d0, bf16_to_f32(yw32[q] & 0xffffu), part);
        part = fmaf(d1, bf16_to_f32(yw32[q] >> 16), part);
        o[2 * q] = wj * d0;
        o[2 * q + 1] = wj * d1;
      }
      *(uint4*)(orow + c * 8) = make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                                           pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) part += __shfl_xor(part, off);
    if (lane == 0) dw[(size_t)t * k + j] = part;
  }
}

// Zero the pad rows [poff[e] + m_e, poff[e+1]) of a padded [rows, H] buffer (block e).
__global__ __launch_bounds__(256) void bwd_zero_pads_kernel(const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ poff,
                                                            uint4* __restrict__ buf, int row_vecs) {
  const int e = blockIdx.x;
  const int m = offsets[e + 1] - offsets[e];
  const int first = poff[e] + max(m, 0), last = poff[e + 1];
  if (last <= first) return;
  const size_t n = (size_t)(last - first) * row_vecs;
  uint4* base = buf + (size_t)first * row_vecs;
  for (size_t i = threadIdx.x; i < n; i += blockDim.x) base[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Router backward, one thread per token, in float64: p = softmax(L); the selected slots S
// (id >= 0, capacity-dropped ones included, with dw = 0); renormalised weights:
// dps_j = (dw_j - sum_i w_i dw_i) / sum_S p, raw: dps_j = dw_j; then
// dL_e = p_e (dp_e - sum_i p_i dp_i) with dp_e = sum of dps_j over slots with id e.
// With the auxiliary load-balancing loss (aux_g != nullptr) every expert's dp_e also gets
// g_e = coeff E f_e / T, the loss's derivative with respect to p[t, e].
template <int KMAX>
__global__ __launch_bounds__(256) void bwd_router_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ topk_idx,
    const float* __restrict__ dw, const double* __restrict__ aux_g, float* __restrict__ dL,
    int T, int E, int k, int renorm) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const float* L = logits + (size_t)t * E;
  double mx = -__builtin_inf();
  for (int e = 0; e < E; ++e) mx = fmax(mx, (double)L[e]);
  double sum = 0.0;
  for (int e = 0; e < E; ++e) sum += exp((double)L[e] - mx);
  int id[KMAX];
  double ps[KMAX], dws[KMAX];
  double s = 0.0, wdw = 0.0;
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    id[j] = -1;
    ps[j] = 0.0;
    dws[j] = 0.0;
    if (j < k) {
      const int e = topk_idx[(size_t)t * k + j];
      if (e >= 0 && e < E) {
        id[j] = e;
        ps[j] = exp((double)L[e] - mx) / sum;
        dws[j] = (double)dw[(size_t)t * k + j];
        s += ps[j];
      }
    }
  }
  if (renorm && s > 0.0) {
#pragma unroll
    for (int j = 0; j < KMAX; ++j) wdw += (ps[j] / s) * dws[j];
#pragma unroll
    for (int j = 0; j < KMAX; ++j) dws[j] = (dws[j] - wdw) / s;
  }
  double dot = 0.0;   // sum_e p_e dp_e
#pragma unroll
  for (int j = 0; j < KMAX; ++j)
    if (id[j] >= 0) dot += ps[j] * dws[j];
  if (aux_g != nullptr)
    for (int e = 0; e < E; ++e) dot += exp((double)L[e] - mx) / sum * aux_g[e];
  for (int e = 0; e < E; ++e) {
    double dp = aux_g != nullptr ? aux_g[e] : 0.0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (id[j] == e) dp += dws[j];
    const double p = exp((double)L[e] - mx) / sum;
    dL[(size_t)t * E + e] = (float)(p * (dp - dot));
  }
}

// Auxiliary load-balancing loss coeff * E * sum_e f_e P_e (the switch-style form; the
// mhpn.cn page's routing chapter adds a loss term that balances the experts' load, the
// lshu.cn page, section 5.3, scales it by moe-aux-loss-coeff), in two deterministic stages.
// Stage 1: block b sums the float64 softmax probabilities of its kAuxTokens tokens per
// expert, in token order.
constexpr int kAuxTokens = 256;
int bwd_aux_blocks(int T) { return (T + kAuxTokens - 1) / kAuxTokens; }

__global__ __launch_bounds__(256) void bwd_aux_partial_kernel(const float* __restrict__ logits,
                                                              double* __restrict__ part, int T,
                                                              int E) {
  __shared__ double smx[kAuxTokens], ssum[kAuxTokens];
  const int t0 = blockIdx.x * kAuxTokens, tid = threadIdx.x;
  const int n = min(kAuxTokens, T - t0);
  if (tid < n) {   // this token's max and partition sum
    const float* L = logits + (size_t)(t0 + tid) * E;
    double mx = -__builtin_inf();
    for (int e = 0; e < E; ++e) mx = fmax(mx, (double)L[e]);
    double sum = 0.0;
    for (int e = 0; e < E; ++e) sum += exp((double)L[e] - mx);
    smx[tid] = mx;
    ssum[tid] = sum;
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    double acc = 0.0;
    for (int i = 0; i < n; ++i)
      acc += exp((double)logits[(size_t)(t0 + i) * E + e] - smx[i]) / ssum[i];
    part[(size_t)blockIdx.x * E + e] = acc;
  }
}

// Stage 2 (one block): P_e = sum of the block partials in block order / T; f_e = counts[e] /
// sum(counts) (pre-capacity counts of the valid selections); g_e = coeff E f_e / T for the
// router backward; loss = coeff E sum_e f_e P_e, summed in expert order.
__global__ __launch_bounds__(256) void bwd_aux_finish_kernel(const double* __restrict__ part,
                                                             int nblocks,
                                                             const int32_t* __restrict__ counts,
                                                             int T, int E, double coeff,
                                                             double* __restrict__ g,
                                                             double* __restrict__ loss) {
  __shared__ double sfp[kMaxExperts];
  __shared__ double sn;
  const int tid = threadIdx.x;
  if (tid == 0) {
    double n = 0.0;
    for (int e = 0; e < E; ++e) n += (double)max(counts[e], 0);
    sn = n;
  }
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    double P = 0.0;
    for (int b = 0; b < nblocks; ++b) P += part[(size_t)b * E + e];
    P /= (double)T;
    const double f = sn > 0.0 ? (double)max(counts[e], 0) / sn : 0.0;
    g[e] = coeff * (double)E * f / (double)T;
    sfp[e] = f * P;
  }
  __syncthreads();
  if (tid == 0) {
    double acc = 0.0;
    for (int e = 0; e < E; ++e) acc += sfp[e];
    *loss = coeff * (double)E * acc;
  }
}

hipError_t launch_bwd_aux_loss(const float* logits, const int32_t* counts, double* part,
                               double* g, double* loss, int T, int E, double coeff,
                               hipStream_t s) {
  const int nb = bwd_aux_blocks(T);
  hipLaunchKernelGGL(bwd_aux_partial_kernel, dim3(nb), dim3(256), 0, s, logits, part, T, E);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(bwd_aux_finish_kernel, dim3(1), dim3(256), 0, s, part, nb, counts, T, E,
                     coeff, g, loss);
  return hipGetLastError();
}

// dx[t] = sum_e dL[t,e] W_router[:, e] + sum over kept slots (slot order) of dxP[padded row],
// float32, one wave per token, 8 columns per lane per vector.
__global__ __launch_bounds__(256) void bwd_dx_kernel(
    const bf16_t* __restrict__ dxP, const bf16_t* __restrict__ w_router,
    const float* __restrict__ dL, const int32_t* __restrict__ slot_row,
    const int32_t* __restrict__ topk_idx, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ poff, bf16_t* __restrict__ dx, int T, int H, int E, int k,
    int nrows, int prows) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  int prow = -1;
  if (lane < k) {
    const int r = slot_row[(size_t)t * k + lane];
    const int e = topk_idx[(size_t)t * k + lane];
    if (r >= 0 && r < nrows && e >= 0 && e < E) prow = r - offsets[e] + poff[e];
    if (prow >= prows) prow = -1;   // inconsistent maps: never read outside dxP
  }
  const float* dl = dL + (size_t)t * E;
  const int nvec = H / 8;
  for (int c = lane; c < nvec; c += 64) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    if ((E & 7) == 0) {   // W_router rows of 8 experts as 16-byte vectors
      for (int e0 = 0; e0 < E; e0 += 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint4 v = *(const uint4*)(w_router + (size_t)(c * 8 + i) * E + e0);
          const uint32_t w32[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            acc[i] = fmaf(dl[e0 + 2 * q], bf16_to_f32(w32[q] & 0xffffu), acc[i]);
            acc[i] = fmaf(dl[e0 + 2 * q + 1], bf16_to_f32(w32[q] >> 16), acc[i]);
          }
        }
      }
    } else {
      for (int e = 0; e < E; ++e) {
        const float g = dl[e];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          acc[i] = fmaf(g, bf16_to_f32(w_router[(size_t)(c * 8 + i) * E + e]), acc[i]);
      }
    }
    for (int j = 0; j < k; ++j) {
      const int pr = __shfl(prow, j);
      if (pr < 0) continue;
      const uint4 v = *(const uint4*)(dxP + (size_t)pr * H + c * 8);
      const uint32_t w32[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_to_f32(w32[q] & 0xffffu);
        acc[2 * q + 1] += bf16_to_f32(w32[q] >> 16);
      }
    }
    *(uint4*)(dx + (size_t)t * H + c * 8) =
        make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

// dW_router = x^T dL and dbias = sum_t dL, in two deterministic stages. Stage 1: block
// (hc, tc) sums tokens [256 tc, 256 tc + 256) for columns [64 hc, 64 hc + 64) of H and all
// experts (16 at a time), four token quarters added in a fixed order; block column hc = 0
// also sums dL for the bias. Stage 2 adds the token-chunk partials in order.
constexpr int kWrTok = 256;
__global__ __launch_bounds__(256) void bwd_wrouter_partial_kernel(
    const bf16_t* __restrict__ x, const float* __restrict__ dL, float* __restrict__ part,
    float* __restrict__ bpart, int T, int H, int E) {
  __shared__ float red[4][64][17];
  const int tid = threadIdx.x, hl = tid & 63, q = tid >> 6;
  const int h = blockIdx.x * 64 + hl, tc = blockIdx.y;
  const int t0 = tc * kWrTok + q * (kWrTok / 4), t1 = min(t0 + kWrTok / 4, T);
  for (int e0 = 0; e0 < E; e0 += 16) {
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    if (h < H)
      for (int t = t0; t < t1; ++t) {
        const float xv = bf16_to_f32(x[(size_t)t * H + h]);
        const float* dl = dL + (size_t)t * E + e0;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (e0 + i < E) acc[i] = fmaf(xv, dl[i], acc[i]);
      }
#pragma unroll
    for (int i = 0; i < 16; ++i) red[q][hl][i] = acc[i];
    __syncthreads();
    if (q == 0 && h < H)
      for (int i = 0; i < 16 && e0 + i < E; ++i)
        part[((size_t)tc * H + h) * E + e0 + i] =
            ((red[0][hl][i] + red[1][hl][i]) + red[2][hl][i]) + red[3][hl][i];
    __syncthreads();
  }
  if (blockIdx.x == 0)
    for (int e = tid; e < E; e += blockDim.x) {
      float sacc = 0.f;
      for (int t = tc * kWrTok; t < min(tc * kWrTok + kWrTok, T); ++t) sacc += dL[(size_t)t * E + e];
      bpart[(size_t)tc * E + e] = sacc;
    }
}

__global__ __launch_bounds__(256) void bwd_wrouter_sum_kernel(
    const float* __restrict__ part, const float* __restrict__ bpart, float* __restrict__ dwr,
    float* __restrict__ dbias, int NC, int H, int E) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < H * E) {
    float s = 0.f;
    for (int c = 0; c < NC; ++c) s += part[(size_t)c * H * E + i];
    dwr[i] = s;
  }
  if (dbias != nullptr && i < E) {
    float s = 0.f;
    for (int c = 0; c < NC; ++c) s += bpart[(size_t)c * E + i];
    dbias[i] = s;
  }
}

// ---------------------------------------------------------------------------------------
int bwd_padded_rows(int T, int k, int E) { return T * k + E * (kPadRows - 1); }

hipError_t launch_bwd_prepare(const bf16_t* x, const int32_t* offsets, const int32_t* row_token,
                              int32_t* poff, int32_t* prow_token, bf16_t* xP,
                              const int32_t* gen, const int32_t* gen_saved, int32_t* bflag,
                              int T, int H, int E, int k, hipStream_t s) {
  const int prows = bwd_padded_rows(T, k, E);
  hipLaunchKernelGGL(bwd_pad_offsets_kernel, dim3(1), dim3(64), 0, s, offsets, poff, E, T * k,
                     gen, gen_saved, bflag);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(bwd_pad_rows_kernel, dim3((prows + 3) / 4), dim3(256), 0, s,
                     (const uint4*)x, offsets, poff, row_token, prow_token, (uint4*)xP, E, T,
                     T * k, prows, H / 8);
  return hipGetLastError();
}

hipError_t launch_bwd_pad_copy(const bf16_t* src, bf16_t* dst, const int32_t* offsets,
                               const int32_t* poff, int T, int k, int E, int row_vecs,
                               hipStream_t s) {
  const int prows = bwd_padded_rows(T, k, E);
  hipLaunchKernelGGL(bwd_pad_copy_kernel, dim3((prows + 3) / 4), dim3(256), 0, s,
                     (const uint4*)src, (uint4*)dst, offsets, poff, E, T * k, prows, row_vecs);
  return hipGetLastError();
}

hipError_t launch_bwd_combine(const bf16_t* dout, const bf16_t* y, const int32_t* slot_row,
                              const int32_t* topk_idx, const float* topk_w,
                              const int32_t* offsets, const int32_t* poff, bf16_t* dyP,
                              float* dw, int T, int H, int E, int k, hipStream_t s) {
  const dim3 grid((T + 3) / 4), block(256);
#define MOE_BC(KM)                                                                           \
  hipLaunchKernelGGL((bwd_combine_kernel<KM>), grid, block, 0, s, dout, y, slot_row, topk_idx, \
                     topk_w, offsets, poff, dyP, dw, T, H, E, k, T * k, bwd_padded_rows(T, k, E))
  if (k <= 2) MOE_BC(2);
  else if (k <= 4) MOE_BC(4);
  else if (k <= 8) MOE_BC(8);
  else MOE_BC(16);
#undef MOE_BC
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(bwd_zero_pads_kernel, dim3(E), dim3(256), 0, s, offsets, poff,
                     (uint4*)dyP, H / 8);
  return hipGetLastError();
}

hipError_t launch_bwd_router(const float* logits, const int32_t* topk_idx, const float* dw,
                             const double* aux_g, float* dL, int T, int E, int k, int renorm,
                             hipStream_t s) {
  const dim3 grid((T + 255) / 256), block(256);
#define MOE_BR(KM) \
  hipLaunchKernelGGL((bwd_router_kernel<KM>), grid, block, 0, s, logits, topk_idx, dw, aux_g, \
                     dL, T, E, k, renorm)
  if (k <= 2) MOE_BR(2);
  else if (k <= 4) MOE_BR(4);
  else if (k <= 8) MOE_BR(8);
  else MOE_BR(16);
#undef MOE_BR
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const bf16_t* dxP, const bf16_t* w_router, const float* dL,
                         const int32_t* slot_row, const int32_t* topk_idx,
                         const int32_t* offsets, const int32_t* poff, bf16_t* dx, int T, int H,
                         int E, int k, hipStream_t s) {
  hipLaunchKernelGGL(bwd_dx_kernel, dim3((T + 3) / 4), dim3(256), 0, s, dxP, w_router, dL,
                     slot_row, topk_idx, offsets, poff, dx, T, H, E, k, T * k,
                     bwd_padded_rows(T, k, E));
  return hipGetLastError();
}

int bwd_wrouter_chunks(int T) { return (T + kWrTok - 1) / kWrTok; }

hipError_t launch_bwd_wrouter(const bf16_t* x, const float* dL, float* part, float* bpart,
                              float* dwr, float* dbias, int T, int H, int E, hipStream_t s) {
  const int NC = bwd_wrouter_chunks(T);
  hipLaunchKernelGGL(bwd_wrouter_partial_kernel, dim3((H + 63) / 64, NC), dim3(256), 0, s, x,
                     dL, part, bpart, T, H, E);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(bwd_wrouter_sum_kernel, dim3((H * E + 255) / 256), dim3(256), 0, s, part,
                     bpart, dwr, dbias, NC, H, E);
  return hipGetLastError();
}


}  // namespace moe
