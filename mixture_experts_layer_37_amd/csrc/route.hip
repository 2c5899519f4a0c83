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
// bf16 path: the gate GEMM runs on MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulation) and
// x is streamed from HBM exactly once. For a small gate (E <= 16) route_stream_kernel
// stages the token rows through LDS in coalesced pieces and keeps the router weight in
// registers; a larger gate is first packed into the workspace as MFMA operands
// (router_pack_kernel) and route_wide_kernel shares each piece of token rows among eight
// waves through LDS.
#include <climits>

#include "common.h"
#include "kernels.h"

namespace moe {

typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// Total order used for selection: -0.0 == +0.0, NaN below -inf, otherwise the float order.
__device__ __forceinline__ int order_key(float f) {
  if (f != f) return INT_MIN + 1;
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) return 0;
  return (u & 0x80000000u) ? (int)(u ^ 0x7fffffffu) : (int)u;
}

// Top-k of one token's E logits (any address space) and its gate weights. Weights are
// evaluated in float64 and rounded once to float32. With `thr`, threshold routing
// (intelliparadigm.com page, section 3.2.1): only the experts whose softmax score exceeds
// `delta` are kept, best first, at most k; the other slots get id -1 and weight 0.
// Returns true if a logit is not finite.
template <int KMAX>
__device__ bool topk_token(const float* L, int E, int k, int renorm, int thr, double delta,
                           int32_t* idx_out, float* w_out, int* ids = nullptr) {
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
  int cnt = k;   // slots that hold an expert
  if (thr) {
    // threshold routing: p_j = exp(L_j - top) / sum over every expert, kept while
    // p_j > delta (p falls along the sorted list, so the kept experts are a prefix)
    double all = 0.0;
    for (int e = 0; e < E; ++e) all += exp((double)L[e] - top);
    cnt = 0;
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      if (j < k) {
        ev[j] = exp((double)L[id[j]] - top);
        if (cnt == j && ev[j] / all > delta) cnt = j + 1;
      }
    if (renorm) {
#pragma unroll
      for (int j = 0; j < KMAX; ++j)
        if (j < cnt) s += ev[j];
    } else {
      s = all;
    }
  } else if (renorm) {
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
    if (j < cnt) {
      idx_out[j] = id[j];
      w_out[j] = has_nan ? __builtin_nanf("") : (float)(ev[j] / s);
    } else if (j < k) {
      idx_out[j] = -1;
      w_out[j] = 0.f;
    }
    if (ids != nullptr) ids[j] = j < cnt ? id[j] : -1;   // what idx_out now holds (-1 past k)
  }
  return nonfinite;
}

int route_padded_experts(int E) {
  return E <= 32 ? 32 : E <= 64 ? 64 : E <= 128 ? 128 : 256;
}

// Router weights W[H][E] -> MFMA B operands in load order: WP[nb][s][l] (16 bytes per lane) =
// W[32 s + 8 (l >> 4) + i][16 nb + (l & 15)], i = 0..7, zero for experts >= E. One k-step's
// operand of 16 experts is then one contiguous 1 KB block. One thread per 16-byte chunk.
__global__ __launch_bounds__(256) void router_pack_kernel(const bf16_t* __restrict__ w,
                                                          bf16_t* __restrict__ wp, int H, int E,
                                                          int EP) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const int S = H / 32;
  if (i >= (long)(EP / 16) * S * 64) return;
  const int l = (int)(i & 63);
  const long bs = i >> 6;
  const int s = (int)(bs % S), nb = (int)(bs / S);
  const int e = nb * 16 + (l & 15);
  const int k0 = s * 32 + 8 * (l >> 4);
  uint32_t d[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t lo = 0, hi = 0;
    if (e < E) {
      lo = w[(size_t)(k0 + 2 * q) * E + e];
      hi = w[(size_t)(k0 + 2 * q + 1) * E + e];
    }
    d[q] = lo | (hi << 16);
  }
  *(uint4*)(wp + i * 8) = make_uint4(d[0], d[1], d[2], d[3]);
}

hipError_t launch_router_pack(const bf16_t* w, bf16_t* wt, int H, int E, hipStream_t s) {
  const int EP = route_padded_experts(E);
  const long n = (long)(EP / 16) * (H / 32) * 64;
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(router_pack_kernel, dim3(blocks), dim3(256), 0, s, w, wt, H, E, EP);
  return hipGetLastError();
}

// DPP lane moves inside rows of 16 lanes (quad_perm and mirror controls).
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
  const unsigned long long u = __double_as_longlong(v);
  const int lo = dpp_i<CTRL>((int)(u & 0xffffffffu)), hi = dpp_i<CTRL>((int)(u >> 32));
  return __longlong_as_double((long long)(((unsigned long long)(unsigned)hi << 32) | (unsigned)lo));
}
// (key, id) pair order of the selection: larger key first, then the lower expert id.
__device__ __forceinline__ bool pair_before(int ka, int ia, int kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}
// Best pair over the 4 lanes of a quad, identical in all of them.
template <int CTRL>
__device__ __forceinline__ void quad_best_step(int& key, int& id) {
  const int ok = dpp_i<CTRL>(key), oi = dpp_i<CTRL>(id);
  if (pair_before(ok, oi, key, id)) { key = ok; id = oi; }
}

// Gate GEMM on MFMA + top-k for gates the streaming router does not take (E up to 256, any
// H that is a multiple of 256). A block of 8 waves owns BT tokens; wave (tw, ew, kw) computes
// TGW token groups of 16 x NBW expert blocks of 16 over its share (1 / KW) of each piece of
// H. Token rows are shared by all waves through LDS: a piece is BT rows x 128 PW k, loaded
// as 16-byte register loads that each cover four whole 256-byte row pieces (fully
// coalesced), written to one of two LDS buffers (16-byte chunk c of row r at c ^ (r & 15):
// conflict-free) and read back as v_mfma_f32_16x16x32_bf16 operands (fp32 accumulation).
// The router weight comes in packed form (router_pack_kernel), one 1 KB load per k-step and
// expert block, straight into registers, from L2 after the first blocks. A piece's rows and
// weights are issued together, D pieces (2 or 4, dividing the piece count) ahead.
// The KW partial sums of a logit are added in a fixed order through LDS (deterministic).
// Selection: 4 lanes per token, each holding every 4th expert; k rounds each take the best
// remaining (key, id) pair of the quad -- so the lower index wins ties, as in topk_token --
// and the weights follow topk_token's formulas in float64, the sums spread over the quad in
// a fixed order.
template <int BT, int TW, int EW, int KW, int NBW, int PW, int D>
__global__ __launch_bounds__(512, 1) void route_wide_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wp, const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ flags, int T, int H, int E, int k, int renorm, int thr, double delta) {
  static_assert(TW * EW * KW == 8, "eight waves");
  static_assert(D == 2 || D == 4, "ring depths the launcher picks");
  constexpr int TGW = BT / (16 * TW);   // token groups per wave
  constexpr int EP = EW * NBW * 16;     // padded experts
  constexpr int SUB = BT * 128;         // elements of one [BT][128] sub-piece
  constexpr int PIECE = SUB * PW;
  constexpr int XL = BT * PW / 32;      // 1 KB x loads per wave per piece
  constexpr int QS = 4 * PW;            // k-steps per piece
  constexpr int QW = QS / KW;           // k-steps per wave per piece
  constexpr int LDL = EP + 1;           // logit tile row stride (floats)
  constexpr int G = 4, EPL = EP / G;    // lanes per token in the selection, experts per lane
  static_assert(TGW >= 1 && XL >= 1 && QW >= 1 && BT <= 128, "block shape");
  __shared__ __attribute__((aligned(1024))) bf16_t xs[2 * PIECE];
  __shared__ float lt[BT * LDL];
  __shared__ int nfs[BT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave % KW, ew = (wave / KW) % EW, tw = wave / (KW * EW);
  const int t0 = blockIdx.x * BT;
  const int S = H / 32;
  const int NP = H / (128 * PW);

  // x loads of this wave: load i covers rows 4 rg .. 4 rg + 3 of sub-piece sp
  const bf16_t* xsrc[XL];
  int xdst[XL];
#pragma unroll
  for (int i = 0; i < XL; ++i) {
    const int gi = wave * XL + i, sp = gi / (BT / 4), rg = gi % (BT / 4);
    const int r = 4 * rg + (lane >> 4), c = lane & 15;
    xsrc[i] = x + (size_t)min(t0 + r, T - 1) * H + sp * 128 + c * 8;
    xdst[i] = sp * SUB + r * 128 + ((c ^ (r & 15)) << 3);
  }
  // packed weight operands of this wave: expert block ew * NBW + j, k-step p * QS + kw * QW + q
  const bf16_t* wsrc[NBW];
#pragma unroll
  for (int j = 0; j < NBW; ++j)
    wsrc[j] = wp + ((size_t)(ew * NBW + j) * S + kw * QW) * 512 + lane * 8;

  bf16x8 xr[D][XL];
  bf16x8 wr[D][QW][NBW];
  auto load_x = [&](int p, bf16x8* v) {
#pragma unroll
    for (int i = 0; i < XL; ++i) v[i] = *(const bf16x8*)(xsrc[i] + (size_t)p * 128 * PW);
  };
  auto load_w = [&](int p, bf16x8 (*v)[NBW]) {
#pragma unroll
    for (int q = 0; q < QW; ++q)
#pragma unroll
      for (int j = 0; j < NBW; ++j) v[q][j] = *(const bf16x8*)(wsrc[j] + ((size_t)p * QS + q) * 512);
  };

  f32x4 acc[TGW][NBW];
#pragma unroll
  for (int g = 0; g < TGW; ++g)
#pragma unroll
    for (int j = 0; j < NBW; ++j) acc[g][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // A wave's vector loads complete in issue order, so piece p's token rows and weights are
  // both issued D pieces ahead (a ring of D register sets): waiting for them never waits for
  // a later piece. Issue order: pieces 0 .. D - 1 (kept by the scheduling barriers), then in
  // step p the rows of piece p + D right after their registers are written to LDS and its
  // weights after the MFMAs that read the set. D divides NP, so the loop body has no branch
  // and every wait is an exact count; prefetches past the last piece re-read it.
#pragma unroll
  for (int u = 0; u < D; ++u) {
    load_x(min(u, NP - 1), xr[u]);
    load_w(min(u, NP - 1), wr[u]);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int p0 = 0; p0 < NP; p0 += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const int p = p0 + u;
      bf16_t* buf = xs + (p & 1) * PIECE;
#pragma unroll
      for (int i = 0; i < XL; ++i) *(bf16x8*)(buf + xdst[i]) = xr[u][i];
      load_x(min(p + D, NP - 1), xr[u]);
      // this piece is in LDS for every wave; every wave is done with the buffer's previous
      // piece (its reads fed MFMAs issued before this point). No wait on the loads in flight.
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
      for (int q = 0; q < QW; ++q) {
        const int qq = kw * QW + q;
        const int sp = qq >> 2, c = 4 * (qq & 3) + (lane >> 4);
        bf16x8 a[TGW];
#pragma unroll
        for (int g = 0; g < TGW; ++g) {
          const int r = (tw * TGW + g) * 16 + (lane & 15);
          a[g] = *(const bf16x8*)(buf + sp * SUB + r * 128 + ((c ^ (r & 15)) << 3));
        }
#pragma unroll
        for (int g = 0; g < TGW; ++g)
#pragma unroll
          for (int j = 0; j < NBW; ++j)
            acc[g][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[g], wr[u][q][j], acc[g][j],
                                                                0, 0, 0);
      }
      load_w(min(p + D, NP - 1), wr[u]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Logit tile [BT][EP]: MFMA 16x16 output, lane holds expert lane & 15 of tokens
  // 4 (lane >> 4) + r. The KW k-shares are added in the order ((kw 0 + kw 1) + kw 2) + ..,
  // then the gate bias.
  auto tile = [&](int g, int j, int r) -> float& {
    return lt[((tw * TGW + g) * 16 + 4 * (lane >> 4) + r) * LDL + (ew * NBW + j) * 16 +
              (lane & 15)];
  };
#pragma unroll
  for (int kk = 1; kk < KW; ++kk) {
    if (kw == kk) {
#pragma unroll
      for (int g = 0; g < TGW; ++g)
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) tile(g, j, r) = acc[g][j][r];
    }
    __syncthreads();
    if (kw == 0) {
#pragma unroll
      for (int g = 0; g < TGW; ++g)
#pragma unroll
        for (int j = 0; j < NBW; ++j)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[g][j][r] += tile(g, j, r);
    }
    __syncthreads();
  }
  if (kw == 0) {
#pragma unroll
    for (int j = 0; j < NBW; ++j) {
      const int e = (ew * NBW + j) * 16 + (lane & 15);
      const float b = (bias != nullptr && e < E) ? bias[e] : 0.f;
#pragma unroll
      for (int g = 0; g < TGW; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) tile(g, j, r) = acc[g][j][r] + b;
    }
  }
  __syncthreads();
  for (int i = tid; i < BT * E; i += blockDim.x) {
    const int tt = i / E, e = i - tt * E;
    if (t0 + tt < T) logits[(size_t)(t0 + tt) * E + e] = lt[tt * LDL + e];
  }

  // Selection and weights: quad (tid >> 2) owns token tt; lane gl holds experts gl + 4 i.
  const int tt = tid >> 2, gl = tid & 3;
  const int t = t0 + tt;
  if (tt < BT) {
    const float* row = lt + tt * LDL;
    int key[EPL];
    int nan_l = 0, nf_l = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const int e = gl + G * i;
      key[i] = INT_MIN;   // below every real key (NaN maps to INT_MIN + 1)
      if (e < E) {
        const float v = row[e];
        key[i] = order_key(v);
        nan_l |= (v != v);
        nf_l |= !__builtin_isfinite(v);
      }
    }
    nan_l |= dpp_i<kDppXor1>(nan_l);
    nan_l |= dpp_i<kDppXor2>(nan_l);
    nf_l |= dpp_i<kDppXor1>(nf_l);
    nf_l |= dpp_i<kDppXor2>(nf_l);
    // k rounds; lane gl keeps the ids of slots gl, gl + 4, ... (k <= 16)
    int sid[4] = {-1, -1, -1, -1};
    int id0 = 0;
    for (int j = 0; j < k; ++j) {
      int bk = INT_MIN, bi = INT_MAX;
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (key[i] > bk) { bk = key[i]; bi = gl + G * i; }   // ascending ids: lowest id wins
      quad_best_step<kDppXor1>(bk, bi);
      quad_best_step<kDppXor2>(bk, bi);
#pragma unroll
      for (int i = 0; i < EPL; ++i)
        if (gl + G * i == bi) key[i] = INT_MIN;
      if (j == 0) id0 = bi;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (j == gl + G * s) sid[s] = bi;
    }
    const double top = (double)row[id0];
    // ev of this lane's slots; sums over the quad in a fixed order
    double ev[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) ev[s] = sid[s] >= 0 ? exp((double)row[sid[s]] - top) : 0.0;
    auto quad_sum = [&](double v) {
      v += dpp_d<kDppXor1>(v);
      return v + dpp_d<kDppXor2>(v);
    };
    double all = 0.0;
    if (thr || !renorm) {
      double a = 0.0;
#pragma unroll
      for (int i = 0; i < EPL; ++i) {
        const int e = gl + G * i;
        if (e < E) a += exp((double)row[e] - top);
      }
      all = quad_sum(a);
    }
    int cnt = k;
    if (thr) {
      // leading slots whose softmax score exceeds delta
      int pass = 0;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (sid[s] >= 0 && ev[s] / all > delta) pass |= 1 << (gl + G * s);
      pass |= dpp_i<kDppXor1>(pass);
      pass |= dpp_i<kDppXor2>(pass);
      cnt = min(k, __builtin_ctz(~pass));
    }
    double ssum;
    if (renorm) {
      double a = 0.0;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (gl + G * s < cnt) a += ev[s];
      ssum = quad_sum(a);
    } else {
      ssum = all;
    }
    if (t < T) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int j = gl + G * s;
        if (j < cnt) {
          topk_idx[(size_t)t * k + j] = sid[s];
          topk_w[(size_t)t * k + j] = nan_l ? __builtin_nanf("") : (float)(ev[s] / ssum);
        } else if (j < k) {
          topk_idx[(size_t)t * k + j] = -1;
          topk_w[(size_t)t * k + j] = 0.f;
        }
      }
    }
    if (gl == 0) nfs[tt] = (t < T) ? nf_l : 0;
  }
  __syncthreads();
  const int ngroups = (T + kRouteFlagGroup - 1) / kRouteFlagGroup;
  constexpr int FG = BT / kRouteFlagGroup;
  if (tid < FG && (t0 / kRouteFlagGroup) + tid < ngroups) {
    int any = 0;
    for (int i = 0; i < kRouteFlagGroup; ++i) any |= nfs[tid * kRouteFlagGroup + i];
    flags[t0 / kRouteFlagGroup + tid] = any ? 2 /* MOE_FLAG_NONFINITE_LOGIT */ : 0;
  }
}

template <int BT, int TW, int EW, int KW, int NBW, int PW>
static hipError_t launch_route_wide(const bf16_t* x, const bf16_t* wp, const float* bias,
                                    float* logits, int32_t* idx, float* w, int32_t* flags, int T,
                                    int H, int E, int k, int renorm, int thr, double delta,
                                    hipStream_t s) {
  const int NP = H / (128 * PW);   // pieces (even); the ring depth divides it
  const dim3 grid((T + BT - 1) / BT), block(512);
#define MOE_ROUTE_WIDE_D(DD)                                                                  \
  hipLaunchKernelGGL((route_wide_kernel<BT, TW, EW, KW, NBW, PW, DD>), grid, block, 0, s, x, wp, \
                     bias, logits, idx, w, flags, T, H, E, k, renorm, thr, delta)
  if (NP % 4 == 0) MOE_ROUTE_WIDE_D(4);
  else MOE_ROUTE_WIDE_D(2);
#undef MOE_ROUTE_WIDE_D
  return hipGetLastError();
}

hipError_t launch_route_bf16(const bf16_t* x, const bf16_t* wt, const float* bias, float* logits,
                             int32_t* idx, float* w, int32_t* flags, int T, int H, int E, int k,
                             int renorm, int thr, double delta, hipStream_t s) {
  if (H % 256 != 0 || k > 16 || k > E) return hipErrorInvalidValue;
#define MOE_ROUTE_WIDE(...) \
  launch_route_wide<__VA_ARGS__>(x, wt, bias, logits, idx, w, flags, T, H, E, k, renorm, thr, delta, s)
  // widest piece (PW x 128 k) that leaves an even number of pieces; H / 128 is even
  const int h128 = H / 128;
  const int pw = h128 % 8 == 0 ? 4 : h128 % 4 == 0 ? 2 : 1;
  switch (route_padded_experts(E)) {
    // BT, TW, EW, KW, NBW, PW
    case 32:
      if (pw == 4) return MOE_ROUTE_WIDE(32, 1, 2, 4, 1, 4);
      if (pw == 2) return MOE_ROUTE_WIDE(32, 1, 2, 4, 1, 2);
      return MOE_ROUTE_WIDE(32, 1, 2, 4, 1, 1);
    case 64:
      if (pw >= 2) return MOE_ROUTE_WIDE(64, 1, 4, 2, 1, 2);
      return MOE_ROUTE_WIDE(64, 1, 4, 2, 1, 1);
    case 128: return MOE_ROUTE_WIDE(128, 1, 8, 1, 1, 1);
    default: return MOE_ROUTE_WIDE(64, 1, 8, 1, 2, 1);
  }
#undef MOE_ROUTE_WIDE
}

// ---------------------------------------------------------------------------------------
// Router for a small gate (E <= 16, H a multiple of 1024 up to 4096, E * H <= 32768). A block of 8 waves
// owns 32 tokens; wave w owns the w-th eighth of H. Each wave
//   - copies its slice of the router weight (contiguous in W[H, E]) into LDS and reads
//     its MFMA operands from there into registers (8 consecutive k of expert lane & 15 per
//     lane; lanes for experts >= E hold zeros), so W is never transposed in memory;
//   - streams its slice of the 32 token rows through two private LDS buffers of
//     32 rows x 128 k, filled by global->LDS DMA in fully coalesced 1 KB pieces (4 rows x
//     256 bytes): token rows are read from HBM exactly once, in whole 128-byte lines;
//   - runs v_mfma_f32_16x16x32_bf16 (fp32 accumulation) on fragments read back from LDS
//     (16-byte chunk c of row r stored at c ^ (r & 15): conflict-free for 16 rows).
// No barrier is needed until the end: each wave only reads what it loaded. The eight
// partial [32 x 16] tiles are then added in a fixed order through LDS (deterministic
// logits), and one lane per token runs the same top-k and weights as the other paths.
constexpr int kRouteWaves = 8;
constexpr int kRouteSubK = 128;                   // k per staged sub-chunk
constexpr int kRouteBufElems = 32 * kRouteSubK;   // one wave's buffer: 32 rows x 128 k
constexpr int kRouteMaxSteps = 16;                // 32-wide k-steps per wave (H <= 4096)
// s_waitcnt immediates (gfx9: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8):
// wait for all but the newest n vector-memory operations / for every LDS operation.
constexpr int wait_vmcnt(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 0xC07F;

bool route_lds_fits(int H, int E) {
  // H / 8 a multiple of 128 and at most 512 wide; a wave's weight slice fits its buffer
  return E <= 16 && H % (kRouteWaves * kRouteSubK) == 0 &&
         H / kRouteWaves / 32 <= kRouteMaxSteps && (H / kRouteWaves) * E <= kRouteBufElems;
}

template <int KMAX>
__global__ __launch_bounds__(512, 1) void route_stream_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ w, const bf16_t* __restrict__ wt,
    const float* __restrict__ bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int32_t* __restrict__ flags, int32_t* __restrict__ cnt_hist, int32_t* __restrict__ cnt_rank,
    int T, int H, int E, int k, int renorm, int thr, double delta) {
  constexpr int BT = kRouteCountTokens, LDR = 17;   // tokens per block
  // Two buffer sets in two distinct LDS objects, so the compiler can tell a DMA into one
  // from reads of the other.
  __shared__ __attribute__((aligned(1024))) bf16_t xb0[kRouteWaves * kRouteBufElems];
  __shared__ __attribute__((aligned(1024))) bf16_t xb1[kRouteWaves * kRouteBufElems];
  __shared__ float red[kRouteWaves][BT * LDR];
  __shared__ float lg[BT * LDR];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * BT;
  const int hs = H / kRouteWaves;        // this wave's slice of H
  const int kbase = wave * hs;
  const int nsteps = hs / 32;            // 32-wide k-steps in the slice
  const int nsub = hs / kRouteSubK;      // staged sub-chunks (4 steps each)

  // DMA of sub-chunk j of this wave's slice into its buffer: instruction i fills rows
  // 4i .. 4i+3; lane l lands at position l & 15 of row 4i + l/16 and loads the row's chunk
  // (l & 15) ^ (row & 15). Rows past T re-read row T-1 (never used).
  const int drow = lane >> 4, dpos = lane & 15;
  auto dma = [&](int j, bf16_t* set) {
    bf16_t* dst = set + wave * kRouteBufElems;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 4 * i + drow;
      const int row = min(t0 + r, T - 1);
      const bf16_t* src = x + (size_t)row * H + kbase + j * kRouteSubK + ((dpos ^ (r & 15)) << 3);
      __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)(dst + i * 512), 16, 0, 0);
    }
  };
  // The MFMA operands of every k-step of the wave's slice (8 consecutive k of expert
  // lane & 15 per lane; zeros for experts >= E) go into registers before the stream starts.
  //   - A packed router weight (wt, launch_router_pack's layout, packed once at load time):
  //     k-step st is one contiguous 1 KB block of expert group 0, one 16-byte load per lane
  //     of a live expert (the block's zeros for experts >= E are not fetched), issued
  //     together and ahead of the first x sub-chunk. Measured as fast as the plain path:
  //     the wait for the weights is latency either way.
  //   - A plain one: the slice is contiguous in W[H, E] (hs * E elements, at most one
  //     buffer). It is DMA'd into the wave's second buffer ahead of the first x sub-chunk;
  //     once it has landed (all but the 8 newest DMA instructions done), the operands are
  //     read from LDS, after which the buffer is free for x.
  const int n = lane & 15;
  const bool live = n < E;
  bf16x8 wf[kRouteMaxSteps];
  if (wt != nullptr) {
    const bf16x8* src = (const bf16x8*)wt + (size_t)(kbase / 32) * 64 + lane;
#pragma unroll
    for (int st = 0; st < kRouteMaxSteps; ++st)
      wf[st] = (st < nsteps && live) ? src[st * 64] : bf16x8{};   // dead lanes load nothing
    dma(0, xb0);
  } else {
    bf16_t* wsl = xb1 + wave * kRouteBufElems;
    const int wchunks = hs * E / 8;                 // 16-byte chunks of the slice
    const int wdma = (wchunks + 63) / 64;           // 1 KB DMA instructions (<= 8)
    const bf16_t* wsrc = w + (size_t)kbase * E;
    for (int i = 0; i < wdma; ++i) {
      const bf16_t* src = wsrc + (size_t)min(i * 64 + lane, wchunks - 1) * 8;
      __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)(wsl + i * 512), 16, 0, 0);
    }
    dma(0, xb0);
    __builtin_amdgcn_s_waitcnt(wait_vmcnt(8));   // the weight slice has landed
#pragma unroll
    for (int st = 0; st < kRouteMaxSteps; ++st) {
      v8i16 v = {};
      if (st < nsteps && live) {
        const bf16_t* p = wsl + (st * 32 + 8 * (lane >> 4)) * E + n;
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (short)p[i * E];
      }
      wf[st] = __builtin_bit_cast(bf16x8, v);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // the weight slice has been read out
  }

  f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  auto compute = [&](int j, const bf16_t* set) {
    const bf16_t* b = set + wave * kRouteBufElems;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = 4 * q + (lane >> 4);
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int r = 16 * g + (lane & 15);
        const bf16x8 a = *(const bf16x8*)(b + r * kRouteSubK + ((c ^ (r & 15)) << 3));
        // k-step j*4 + q of the slice; the weight operand array is indexed statically
        bf16x8 wv = wf[0];
#pragma unroll
        for (int st = 1; st < kRouteMaxSteps; ++st)
          if (st == j * 4 + q) wv = wf[st];
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, wv, acc[g], 0, 0, 0);
      }
    }
  };

  // Wait for all but the newest DMA batch (8 instructions) or for everything.
  auto wait_dma = [&](bool one_more_in_flight) {
    if (one_more_in_flight) __builtin_amdgcn_s_waitcnt(wait_vmcnt(8));
    else __builtin_amdgcn_s_waitcnt(wait_vmcnt(0));
  };
  if (nsub > 1) dma(1, xb1);
  for (int j = 0; j < nsub; j += 2) {
    // sub-chunk j is in xb0; sub-chunk j + 1 (if any) is in flight into xb1
    wait_dma(j + 1 < nsub);
    compute(j, xb0);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);   // reads of xb0 done
    if (j + 2 < nsub) dma(j + 2, xb0);
    if (j + 1 < nsub) {
      wait_dma(j + 2 < nsub);
      compute(j + 1, xb1);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      if (j + 3 < nsub) dma(j + 3, xb1);
    }
  }

  // MFMA 16x16 output: lane holds expert lane & 15 of tokens 4 (lane >> 4) + r.
#pragma unroll
  for (int g = 0; g < 2; ++g)
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][(g * 16 + 4 * (lane >> 4) + r) * LDR + n] = acc[g][r];
  __syncthreads();
  // Fixed-order sum of the eight partial tiles, plus the gate bias.
  for (int i = tid; i < BT * E; i += blockDim.x) {
    const int tt = i / E, e = i - tt * E;
    float sum = red[0][tt * LDR + e];
#pragma unroll
    for (int v = 1; v < kRouteWaves; ++v) sum += red[v][tt * LDR + e];
    sum += bias != nullptr ? bias[e] : 0.f;
    lg[tt * LDR + e] = sum;
    if (t0 + tt < T) logits[(size_t)(t0 + tt) * E + e] = sum;
  }
  __syncthreads();
  if (tid < 64) {
    bool nf = false;
    const int t = t0 + tid;
    int ev[KMAX];   // this token's ids as written (-1: empty slot or no token)
#pragma unroll
    for (int j = 0; j < KMAX; ++j) ev[j] = -1;
    if (tid < BT && t < T)
      nf = topk_token<KMAX>(lg + tid * LDR, E, k, renorm, thr, delta, topk_idx + (size_t)t * k,
                            topk_w + (size_t)t * k, ev);
    const unsigned long long m = __ballot(nf);
    const int ngroups = (T + kRouteFlagGroup - 1) / kRouteFlagGroup;
    if (tid < 2 && blockIdx.x * 2 + tid < ngroups)
      flags[blockIdx.x * 2 + tid] =
          ((m >> (16 * tid)) & 0xffffull) ? 2 /* MOE_FLAG_NONFINITE_LOGIT */ : 0;
    if (cnt_hist != nullptr) {
      // The permutation's count step for this block's 32 tokens (one count block): per
      // expert, the number of its assignments, and each slot's rank among them in token
      // order. Lane tid holds token t0 + tid; its ids are distinct, in [0, E) or -1 (an empty
      // slot of threshold routing: rank -1, dropped like the count kernel drops it).
      const bool live = tid < BT && t < T;
      int rk[KMAX];
#pragma unroll
      for (int j = 0; j < KMAX; ++j) rk[j] = -1;
      const unsigned long long below = (1ull << tid) - 1ull;
      for (int e = 0; e < E; ++e) {
        bool has = false;
#pragma unroll
        for (int j = 0; j < KMAX; ++j) has |= ev[j] == e;
        const unsigned long long me = __ballot(has);
        if (tid == 0) cnt_hist[(size_t)blockIdx.x * E + e] = (int)__popcll(me);
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (ev[j] == e) rk[j] = (int)__popcll(me & below);
      }
      if (live) {
#pragma unroll
        for (int j = 0; j < KMAX; ++j)
          if (j < k) cnt_rank[(size_t)t * k + j] = rk[j];
      }
    }
  }
}

hipError_t launch_route_bf16_lds(const bf16_t* x, const bf16_t* w_router, const bf16_t* wt,
                                 const float* bias, float* logits, int32_t* idx, float* w,
                                 int32_t* flags, int32_t* cnt_hist, int32_t* cnt_rank, int T,
                                 int H, int E, int k, int renorm, int thr, double delta, int cus,
                                 hipStream_t s) {
  (void)cus;
  const dim3 grid((T + kRouteCountTokens - 1) / kRouteCountTokens), block(64 * kRouteWaves);
#define MOE_ROUTE_STREAM(KM)                                                                    \
  hipLaunchKernelGGL((route_stream_kernel<KM>), grid, block, 0, s, x, w_router, wt, bias, logits, idx, \
                     w, flags, cnt_hist, cnt_rank, T, H, E, k, renorm, thr, delta)
  if (k <= 1) MOE_ROUTE_STREAM(1);
  else if (k <= 2) MOE_ROUTE_STREAM(2);
  else if (k <= 4) MOE_ROUTE_STREAM(4);
  else if (k <= 8) MOE_ROUTE_STREAM(8);
  else MOE_ROUTE_STREAM(16);
#undef MOE_ROUTE_STREAM
  return hipGetLastError();
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
                                                        int E, int k, int renorm, int thr,
                                                        double delta) {
  const int t = blockIdx.x * 64 + threadIdx.x;
  bool nf = false;
  if (t < T)
    nf = topk_token<KMAX>(logits + (size_t)t * E, E, k, renorm, thr, delta, idx + (size_t)t * k,
                          w + (size_t)t * k);
  const unsigned long long m = __ballot(nf);
  const int ngroups = (T + kRouteFlagGroup - 1) / kRouteFlagGroup;
  const int g = blockIdx.x * 4 + threadIdx.x;
  if (threadIdx.x < 4 && g < ngroups)
    flags[g] = ((m >> (16 * threadIdx.x)) & 0xffffull) ? 2 /* MOE_FLAG_NONFINITE_LOGIT */ : 0;
}

hipError_t launch_route_topk(const float* logits, int32_t* idx, float* w, int32_t* flags, int T,
                             int E, int k, int renorm, int thr, double delta, hipStream_t s) {
  const dim3 grid((T + 63) / 64), block(64);
#define MOE_TOPK_LAUNCH(KM) \
  hipLaunchKernelGGL((route_topk_kernel<KM>), grid, block, 0, s, logits, idx, w, flags, T, E, k, \
                     renorm, thr, delta)
  if (k <= 1) MOE_TOPK_LAUNCH(1);
  else if (k <= 2) MOE_TOPK_LAUNCH(2);
  else if (k <= 4) MOE_TOPK_LAUNCH(4);
  else if (k <= 8) MOE_TOPK_LAUNCH(8);
  else MOE_TOPK_LAUNCH(16);
#undef MOE_TOPK_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
