// Achievable-peak probes used by the benchmark to put its roofline fractions next to what
// this device actually sustains: an MFMA-only loop (bf16 dense rate) and a streaming copy
// (HBM bandwidth). Built into libmoe_peaks.so, separate from the layer's library.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace {

using moe::bf16x8;
using moe::f32x16;
using moe::u32x4;

// Each wave runs 8 independent accumulation chains of v_mfma_f32_32x32x16_bf16 on register
// operands (no memory traffic in the loop); 8 chains keep the MFMA pipe busy despite the
// dependent-issue latency of each chain. Launched with one block (one wave per SIMD) per CU,
// as the packed GEMMs run, it issues at ~96% of the nominal per-cycle rate; more waves per
// SIMD contend and sustain less.
__global__ __launch_bounds__(256) void peak_mfma_kernel(float* __restrict__ sink, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(lane - i));
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0];
  sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Streaming copy with nontemporal 16-byte accesses: block b copies 32 KB chunks b, b + grid,
// ... (256 threads x 8 vectors, all 8 loads in flight before the stores). On this device the
// contiguous chunks and the nontemporal hint each raise the sustained rate over a
// grid-stride loop.
__global__ __launch_bounds__(256) void peak_copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, size_t nchunks) {
  constexpr int U = 8;
  for (size_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const size_t base = c * (256 * U) + threadIdx.x;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + base + u * 256);
#pragma unroll
    for (int u = 0; u < U; ++u) __builtin_nontemporal_store(v[u], dst + base + u * 256);
  }
}

// One pass over `n16` 16-byte chunks, grid-stride, eight loads in flight per thread; the
// XOR of what each thread read goes to `sink` so that no load is dropped.
__global__ __launch_bounds__(256) void peak_read_kernel(const u32x4* __restrict__ src,
                                                        size_t n16, unsigned* __restrict__ sink) {
  constexpr int U = 8;
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * blockDim.x * U;
  for (size_t base = (size_t)blockIdx.x * blockDim.x * U + threadIdx.x; base < n16;
       base += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = base + (size_t)u * blockDim.x;
      v[u] = i < n16 ? src[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u];
  }
  sink[blockIdx.x * blockDim.x + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

// MFMA-only loop: `blocks` blocks of 256 threads, `iters` iterations of 8 MFMAs per wave;
// performs blocks * 4 * iters * 8 * 32768 flops. `sink` holds blocks * 256 floats.
int moe_peak_mfma(float* sink, int blocks, int iters, void* stream) {
  if (sink == nullptr || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(peak_mfma_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream, sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// Copy `bytes` (a multiple of 32768) from src to dst (16-byte aligned device buffers).
int moe_peak_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (src == nullptr || dst == nullptr || bytes % 32768 != 0 ||
      ((uintptr_t)src | (uintptr_t)dst) % 16)
    return 1;
  hipLaunchKernelGGL(peak_copy_kernel, dim3(2048), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, (u32x4*)dst, bytes / 32768);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

// Read `bytes` (a multiple of 16) of src once: `blocks` blocks of 256 threads; `sink` holds
// blocks * 256 words.
int moe_peak_read(const void* src, size_t bytes, unsigned* sink, int blocks, void* stream) {
  if (src == nullptr || sink == nullptr || blocks < 1 || bytes % 16 != 0 ||
      (uintptr_t)src % 16)
    return 1;
  hipLaunchKernelGGL(peak_read_kernel, dim3(blocks), dim3(256), 0, (hipStream_t)stream,
                     (const u32x4*)src, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
