// Combine: out[t] = sum_j w[t,j] * y_perm[slot_row[t,j]] over the kept slots.
//
// The pages add expert outputs into the dense output with atomics (hnwysp.cn/news/132341,
// section 2.2, "Atomic Add"; gitcode.csdn.net MoE page, SparseScatterAdd). Here each token
// gathers its k expert rows instead: one wave per token, float32 accumulation in slot
// order, one write per output row, so the result is bit-reproducible and no atomics are
// needed (lshu.cn/news/82007, section 4, npu_moe_token_postprocess restores token order).
#include "common.h"
#include "kernels.h"

namespace moe {

// 8 elements per 16-byte (bf16) or 32-byte (f32) vector.
template <typename T> struct Vec8;
template <> struct Vec8<bf16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *(const uint4*)p; }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = (&v.x)[i >> 1];
    return bf16_to_f32((i & 1) ? (w >> 16) : (w & 0xffffu));
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* a) {
    *(uint4*)p = make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]),
                            pack_bf16x2(a[4], a[5]), pack_bf16x2(a[6], a[7]));
  }
};
template <> struct Vec8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *(const float4*)p;
    b = *(const float4*)(p + 4);
  }
  __device__ __forceinline__ float get(int i) const {
    return i < 4 ? (&a.x)[i] : (&b.x)[i - 4];
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
    *(float4*)(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
};

// out row = sum over the first n of NR compacted slots (rows[j], ws[j]) of ws[j] * y[rows[j]],
// float32, in slot order; U vectors of 8 columns per lane per step, so up to NR * U loads
// are in flight per lane.
template <typename T, int NR, int U>
__device__ __forceinline__ void combine_rows(const T* __restrict__ y, const int* rows,
                                             const float* ws, int n, T* __restrict__ o,
                                             int nvec, int H, int lane) {
  for (int base = 0; base < nvec; base += 64 * U) {
    Vec8<T> v[NR][U];
#pragma unroll
    for (int j = 0; j < NR; ++j)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = base + u * 64 + lane;
        if (j < n && c < nvec) v[j][u].load(y + (size_t)rows[j] * H + c * 8);
      }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = base + u * 64 + lane;
      if (c >= nvec) continue;
      float acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
      for (int j = 0; j < NR; ++j)
        if (j < n)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = fmaf(ws[j], v[j][u].get(i), acc[i]);
      Vec8<T>::store(o + c * 8, acc);
    }
  }
}

// One wave per token. The token's kept slots (row >= 0) are first compacted to the front,
// in slot order, so empty or dropped slots (threshold routing, capacity) cost no load
// slots; the row loop is then sized by the number kept.
template <typename T, int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const T* __restrict__ y,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ topk_w,
                                                      T* __restrict__ out, int Tn, int H, int k,
                                                      int nrows) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= Tn) return;
  int row = -1;
  float w = 0.f;
  if (lane < k) {
    row = slot_row[(size_t)t * k + lane];
    w = topk_w[(size_t)t * k + lane];
    if (row >= nrows) row = -1;   // a row outside y_perm is never read
  }
  unsigned long long kept = __ballot(row >= 0);
  const int n = __popcll(kept);
  int rows[KMAX];
  float ws[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int src = kept ? __builtin_ctzll(kept) : 0;   // lane of the j-th kept slot
    kept &= kept - 1;
    rows[j] = __shfl(row, src);
    ws[j] = __shfl(w, src);
  }
  const int nvec = H / 8;
  T* o = out + (size_t)t * H;
  if (n <= 2 || KMAX <= 2) combine_rows<T, (KMAX < 2 ? KMAX : 2), (KMAX < 2 ? 8 : 4)>(y, rows, ws, n, o, nvec, H, lane);
  else if (n <= 4 || KMAX <= 4) combine_rows<T, (KMAX < 4 ? KMAX : 4), 2>(y, rows, ws, n, o, nvec, H, lane);
  else combine_rows<T, KMAX, 1>(y, rows, ws, n, o, nvec, H, lane);
}

template <typename T>
static hipError_t launch_combine_t(const T* y, const int32_t* slot_row, const float* w, T* out,
                                   int Tn, int H, int k, hipStream_t s) {
  const dim3 grid((Tn + 3) / 4), block(256);
#define MOE_COMBINE(KM) \
  hipLaunchKernelGGL((combine_kernel<T, KM>), grid, block, 0, s, y, slot_row, w, out, Tn, H, k, Tn * k)
  if (k <= 1) MOE_COMBINE(1);
  else if (k <= 2) MOE_COMBINE(2);
  else if (k <= 4) MOE_COMBINE(4);
  else if (k <= 8) MOE_COMBINE(8);
  else MOE_COMBINE(16);
#undef MOE_COMBINE
  return hipGetLastError();
}

hipError_t launch_combine(int dtype_bf16, const void* y, const int32_t* slot_row,
                          const float* topk_w, void* out, int T, int H, int k, hipStream_t s) {
  if (dtype_bf16)
    return launch_combine_t<bf16_t>((const bf16_t*)y, slot_row, topk_w, (bf16_t*)out, T, H, k, s);
  return launch_combine_t<float>((const float*)y, slot_row, topk_w, (float*)out, T, H, k, s);
}

}  // namespace moe
