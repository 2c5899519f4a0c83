// Permute: group the (token, slot) assignments by expert, in token order, apply the
// capacity clamp and gather the token rows (gitcode.csdn.net, "ops-transformer 仓库 - MoE
// 算子优化实战": a per-expert mask feeds SparseGather, and sparse data is kept CSR-style;
// lshu.cn/news/82007, section 4: npu_moe_token_preprocess reorders the tokens).
//
// No float and no global atomics. Three launches; for the row maps only (no x_perm
// destination, for a GEMM that gathers token rows itself) on a batch of at most
// kMapsMaxBlocks count blocks, two: the count, then permute_scan_rows_kernel, in which every
// block does the scan itself from the histogram table and writes its own tokens' rows.
//   count  -- 1024 tokens per block. Per wave and expert a 64-bit lane mask (LDS OR);
//             popcounts give the block's per-expert histogram and each assignment's rank
//             inside the block in token order. Invalid or repeated ids are dropped, flagged
//             (-1, an empty slot of threshold routing, is dropped silently).
//   scan   -- one block: per expert, exclusive prefix over the count blocks (in place),
//             pre-capacity counts, kept = min(count, C), and the kept offsets (a scan over E).
//             It also advances the workspace's permutation generation (and, for a training
//             forward, records it beside the saved pre-activations), so a backward can tell
//             whether the pre-activations it is handed belong to the latest permutation.
//   gather -- one wave per token: row = offsets[e] + block prefix + in-block rank, kept iff
//             below C; writes slot_row / row_token and copies the token row once into each
//             of its kept rows with 16-byte loads and stores, all loads of a chunk in
//             flight together.
#include <atomic>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace moe {

int permute_count_blocks(int T) { return (T + kCountBlockTokens - 1) / kCountBlockTokens; }

__global__ __launch_bounds__(1024) void permute_count_kernel(const int32_t* __restrict__ idx,
                                                             int32_t* __restrict__ hist,
                                                             int32_t* __restrict__ slot_row,
                                                             int32_t* __restrict__ flags, int T,
                                                             int E, int k) {
  constexpr int NW = kCountBlockTokens / kWave;   // 16 waves
  __shared__ unsigned long long masks[NW * kMaxExperts];
  __shared__ int wpre[NW * kMaxExperts];
  __shared__ int sbad;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < NW * E; i += blockDim.x) masks[i] = 0ull;
  if (tid == 0) sbad = 0;
  __syncthreads();

  const int t = blockIdx.x * kCountBlockTokens + tid;
  int ev[kMaxTopK];
  unsigned valid = 0u;
  bool bad = false;
  if (t < T) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        const int e = idx[(size_t)t * k + j];
        bool ok = (unsigned)e < (unsigned)E;
#pragma unroll
        for (int jj = 0; jj < j; ++jj) ok &= (ev[jj] != e);
        ev[j] = e;
        if (ok) {
          valid |= 1u << j;
          atomicOr(&masks[wave * E + e], 1ull << lane);
        } else if (e != -1) {   // -1 marks an empty slot: dropped without a flag
          bad = true;
        }
      }
    }
  }
  if (bad) sbad = 1;
  __syncthreads();
  for (int e = tid; e < E; e += blockDim.x) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      wpre[w * E + e] = run;
      run += __popcll(masks[w * E + e]);
    }
    hist[(size_t)blockIdx.x * E + e] = run;
  }
  __syncthreads();
  if (t < T) {
    const unsigned long long below = (1ull << lane) - 1ull;
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        int r = -1;
        if (valid & (1u << j)) {
          const int e = ev[j];
          r = wpre[wave * E + e] + __popcll(masks[wave * E + e] & below);
        }
        slot_row[(size_t)t * k + j] = r;
      }
    }
  }
  if (tid == 0) flags[blockIdx.x] = sbad ? 1 /* MOE_FLAG_BAD_INDEX */ : 0;
}

// flag_out (may be null): receives the OR of the count blocks' flags.
__global__ __launch_bounds__(256) void permute_scan_kernel(int32_t* __restrict__ hist,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets, int NB,
                                                           int E, int cap, int32_t* gen,
                                                           int32_t* gen_copy,
                                                           const int32_t* __restrict__ flags,
                                                           int32_t* __restrict__ flag_out) {
  __shared__ int wsum[4];
  __shared__ int wflag[4];
  const int e = threadIdx.x, wave = e >> 6, lane = e & 63;
  if (e == 0 && gen != nullptr) {
    const int g = gen[0] + 1;
    gen[0] = g;
    if (gen_copy != nullptr) gen_copy[0] = g;
  }
  if (flag_out != nullptr) {   // uniform branch: every thread takes part
    int f = 0;
    for (int b = e; b < NB; b += blockDim.x) f |= flags[b];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) f |= __shfl_xor(f, o);
    if (lane == 0) wflag[wave] = f;
    __syncthreads();
    if (e == 0) flag_out[0] = wflag[0] | wflag[1] | wflag[2] | wflag[3];
  }
  int run = 0;
  if (e < E) {
    int b = 0;
    for (; b + 8 <= NB; b += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = hist[(size_t)(b + u) * E + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        hist[(size_t)(b + u) * E + e] = run;
        run += v[u];
      }
    }
    for (; b < NB; ++b) {
      const int v = hist[(size_t)b * E + e];
      hist[(size_t)b * E + e] = run;
      run += v;
    }
    counts[e] = run;
  }
  const int kept = e < E ? min(run, cap) : 0;
  int incl = kept;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o);
    if (lane >= o) incl += n;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int pre = 0;
  for (int w = 0; w < wave; ++w) pre += wsum[w];
  incl += pre;
  if (e < E) offsets[e] = incl - kept;
  if (e == E - 1) offsets[E] = incl;
}

template <int U>
__global__ __launch_bounds__(256) void permute_gather_kernel(
    const uint4* __restrict__ x, const int32_t* __restrict__ idx, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ row_token, const int32_t* __restrict__ prefix,
    const int32_t* __restrict__ offsets, uint4* __restrict__ x_perm, int T, int E, int k, int cap,
    int row_vecs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  int row = -1;
  if (lane < k) {
    const int r = slot_row[(size_t)t * k + lane];
    if (r >= 0) {
      const int e = idx[(size_t)t * k + lane];
      const int pos = prefix[(size_t)(t / kCountBlockTokens) * E + e] + r;
      if (pos < cap) row = offsets[e] + pos;
    }
    slot_row[(size_t)t * k + lane] = row;
    if (row >= 0) row_token[row] = t;
  }
  // Copy the token row into each kept destination row (lane j holds slot j's row; the
  // rows are read out one slot at a time as wave-uniform values). Whole chunks of
  // 64 * U 16-byte vectors first, with all U loads in flight, then the remainder. The
  // x_perm rows are written with nontemporal stores (measured faster; nontemporal loads of
  // x were slower).
  const uint4* src = x + (size_t)t * row_vecs;
  int base = 0;
  for (; base + 64 * U <= row_vecs; base += 64 * U) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[base + u * 64 + lane];
    for (int j = 0; j < k; ++j) {
      const int r = __builtin_amdgcn_readlane(row, j);
      if (r < 0) continue;
      uint4* dst = x_perm + (size_t)r * row_vecs + base + lane;
#pragma unroll
      for (int u = 0; u < U; ++u) st_stream(dst + u * 64, v[u]);
    }
  }
  for (int c = base + lane; c < row_vecs; c += 64) {
    const uint4 v = src[c];
    for (int j = 0; j < k; ++j) {
      const int r = __builtin_amdgcn_readlane(row, j);
      if (r >= 0) st_stream(x_perm + (size_t)r * row_vecs + c, v);
    }
  }
}

// Index-only gather: the rows of each slot and the row -> token map, no row copy (for a
// grouped GEMM that reads token rows in place). One thread per token.
__global__ __launch_bounds__(256) void permute_rows_kernel(
    const int32_t* __restrict__ idx, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ row_token, const int32_t* __restrict__ prefix,
    const int32_t* __restrict__ offsets, int T, int E, int k, int cap) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  for (int j = 0; j < k; ++j) {
    int row = -1;
    const int r = slot_row[(size_t)t * k + j];
    if (r >= 0) {
      const int e = idx[(size_t)t * k + j];
      const int pos = prefix[(size_t)(t / kCountBlockTokens) * E + e] + r;
      if (pos < cap) row = offsets[e] + pos;
    }
    slot_row[(size_t)t * k + j] = row;
    if (row >= 0) row_token[row] = t;
  }
}

// The scan and the row maps in one launch (no x_perm), after the count step, for batches
// of at most kMapsMaxBlocks count blocks of the count kernel (CB = kCountBlockTokens) or
// kRoutedMaxBlocks of the streaming router (CB = kRouteCountTokens). A block of 256 threads
// owns 256 tokens; every block reads the whole [NB][E] histogram table and derives from
// it, in the scan kernel's order, each expert's pre-capacity count, kept offsets and the
// prefix over the count blocks before each of its tokens' own, so no block waits for
// another. Block 0 writes counts and offsets, advances the generation and gathers the flag
// words (after the router's count, which raises none: clears them); every block then turns
// its tokens' in-block ranks (slot_row, from the count step) into rows, as the rows kernel
// does, with all of a token's slot loads in flight together.
static_assert(kCountBlockTokens % 256 == 0, "a 256-token block lies in one count block");
static_assert(256 % kRouteCountTokens == 0, "a 256-token block holds whole router blocks");
constexpr int kRoutedExperts = 16;   // the streaming router's gates: E <= 16
template <int CB>
__global__ __launch_bounds__(256) void permute_scan_rows_kernel(
    const int32_t* __restrict__ idx, const int32_t* __restrict__ hist,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
    int32_t* __restrict__ slot_row, int32_t* __restrict__ flags, int32_t* gen,
    int32_t* gen_copy, int32_t* __restrict__ flag_out, int T, int E, int k, int cap) {
  constexpr bool kRouted = CB == kRouteCountTokens;
  constexpr int kLocal = kRouted ? 256 / CB : 1;   // count blocks a block's tokens span
  // assignments of earlier count blocks, per local count block and expert
  __shared__ int before[kLocal][kRouted ? kRoutedExperts : kMaxExperts];
  __shared__ int red[kRouted ? 2 * 256 : 1];                   // partial sums per reducer
  __shared__ int loc[kLocal][kRouted ? kRoutedExperts : 1];   // the block's own table rows
  __shared__ int tab[kRouted ? 256 * kRoutedExperts : 1];     // 256 rows of the table
  __shared__ int off[kMaxExperts + 1];
  __shared__ int wsum[4];
  __shared__ int wflag[4];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int t = blockIdx.x * blockDim.x + tid;
  const int NB = (T + CB - 1) / CB;
  // this thread's token: its slots' in-block ranks and ids, all loads in flight together
  // (issued first: they land while the histogram table is read)
  int r[kMaxTopK], ev[kMaxTopK];
  if (t < T) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j < k) {
        r[j] = slot_row[(size_t)t * k + j];
        ev[j] = idx[(size_t)t * k + j];
      }
  }
  int total = 0;
  if constexpr (!kRouted) {
    // expert tid: the prefix over count blocks < cb and the batch total
    const int cb = (blockIdx.x * blockDim.x) / CB;   // this block's count block
    if (tid < E) {
      int pre = 0, ob = 0;
      for (; ob + 8 <= NB; ob += 8) {
        int v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = hist[(size_t)(ob + u) * E + tid];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          pre += ob + u < cb ? v[u] : 0;
          total += v[u];
        }
      }
      for (; ob < NB; ++ob) {
        const int v = hist[(size_t)ob * E + tid];
        pre += ob < cb ? v : 0;
        total += v;
      }
      before[0][tid] = pre;
    }
  } else {
    // Many small count blocks. The table goes through LDS 256 rows at a time (coalesced
    // loads); thread (g, e), g < G = 256 / E, sums rows g, g + G, ... of each piece for expert
    // e, over the rows before this block's first count block b0 and over all rows; the G
    // partial sums of each expert are then added. The block's own kLocal rows go to LDS beside, for
    // the prefix inside the block.
    const int b0 = blockIdx.x * kLocal;
    if (tid < kLocal * E) {
      const int c = tid / E, e = tid - c * E;
      loc[c][e] = b0 + c < NB ? hist[(size_t)(b0 + c) * E + e] : 0;
    }
    int pre = 0, tot = 0;
    const int G = 256 / E;                    // reducers per expert
    const int g = tid / E, e = tid - g * E;   // reducer (g, e) for tid < G E
    for (int base = 0; base < NB; base += 256) {
      const int rows = min(256, NB - base);
      int v[kRoutedExperts];   // all of this thread's loads in flight together
#pragma unroll
      for (int u = 0; u < kRoutedExperts; ++u) {
        const int i = tid + u * 256;
        v[u] = i < rows * E ? hist[(size_t)base * E + i] : 0;
      }
#pragma unroll
      for (int u = 0; u < kRoutedExperts; ++u)
        if (tid + u * 256 < rows * E) tab[tid + u * 256] = v[u];
      __syncthreads();
      if (tid < G * E) {
#pragma unroll 4
        for (int rr = g; rr < rows; rr += G) {
          const int x = tab[rr * E + e];
          tot += x;
          pre += base + rr < b0 ? x : 0;
        }
      }
      __syncthreads();
    }
    if (tid < G * E) {
      red[tid] = pre;
      red[256 + tid] = tot;
    }
    __syncthreads();
    // local count block c (tid / E), expert e: the prefix before b0 plus rows b0 .. b0 + c - 1
    if (tid < kLocal * E) {
      const int c = tid / E, ee = tid - c * E;
      int p = 0;
#pragma unroll 8
      for (int gg = 0; gg < G; ++gg) p += red[gg * E + ee];
      for (int cc = 0; cc < c; ++cc) p += loc[cc][ee];
      before[c][ee] = p;
    }
    if (tid < E) {
#pragma unroll 8
      for (int gg = 0; gg < G; ++gg) total += red[256 + gg * E + tid];
    }
  }
  // exclusive scan of min(total, cap) over E <= 256 experts (one per thread)
  const int kept = tid < E ? min(total, cap) : 0;
  int incl = kept;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o);
    if (lane >= o) incl += n;
  }
  if (lane == 63) wsum[wave] = incl;
  // block 0: the OR of the count blocks' flag words (after the router's count: none, and
  // the count kernel's words are cleared)
  int f = 0;
  if constexpr (!kRouted) {
    if (blockIdx.x == 0 && flag_out != nullptr)
      for (int ob = tid; ob < NB; ob += blockDim.x) f |= flags[ob];
  } else {
    if (blockIdx.x == 0)
      for (int ob = tid; ob < (T + kCountBlockTokens - 1) / kCountBlockTokens; ob += blockDim.x)
        flags[ob] = 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) f |= __shfl_xor(f, o);
  if (lane == 0) wflag[wave] = f;
  __syncthreads();
  {
    int pre = 0;
    for (int w = 0; w < wave; ++w) pre += wsum[w];
    incl += pre;
    if (tid < E) off[tid] = incl - kept;
    if (tid == E - 1) off[E] = incl;
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    if (tid < E) counts[tid] = total;
    for (int e = tid; e <= E; e += blockDim.x) offsets[e] = off[e];
    if (tid == 0) {
      if (gen != nullptr) {
        const int g = gen[0] + 1;
        gen[0] = g;
        if (gen_copy != nullptr) gen_copy[0] = g;
      }
      if (flag_out != nullptr) flag_out[0] = wflag[0] | wflag[1] | wflag[2] | wflag[3];
    }
  }
  if (t < T) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < k) {
        int row = -1;
        if (r[j] >= 0) {
          const int pos = before[kRouted ? tid / CB : 0][ev[j]] + r[j];
          if (pos < cap) row = off[ev[j]] + pos;
        }
        slot_row[(size_t)t * k + j] = row;
        if (row >= 0) row_token[row] = t;
      }
    }
  }
}

hipError_t launch_permute(const void* x, int elem_bytes, const int32_t* topk_idx, void* x_perm,
                          int32_t* counts, int32_t* offsets, int32_t* row_token,
                          int32_t* slot_row, int32_t* hist, int32_t* flags, int32_t* gen,
                          int32_t* gen_copy, int32_t* flag_out, int T, int H, int E, int k,
                          int cap, hipStream_t s) {
  const int NB = permute_count_blocks(T);
  hipLaunchKernelGGL(permute_count_kernel, dim3(NB), dim3(kCountBlockTokens), 0, s, topk_idx,
                     hist, slot_row, flags, T, E, k);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (x_perm == nullptr && NB <= kMapsMaxBlocks) {
    hipLaunchKernelGGL(permute_scan_rows_kernel<kCountBlockTokens>, dim3((T + 255) / 256),
                       dim3(256), 0, s, topk_idx, hist, counts, offsets, row_token, slot_row,
                       flags, gen, gen_copy, flag_out, T, E, k, cap);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(256), 0, s, hist, counts, offsets, NB, E,
                     cap, gen, gen_copy, flags, flag_out);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (x_perm == nullptr) {
    hipLaunchKernelGGL(permute_rows_kernel, dim3((T + 255) / 256), dim3(256), 0, s, topk_idx,
                       slot_row, row_token, hist, offsets, T, E, k, cap);
    return hipGetLastError();
  }
  const int row_vecs = (int)((size_t)H * elem_bytes / 16);
  const dim3 grid((T + 3) / 4), block(256);
#define MOE_GATHER(U_)                                                                      \
  hipLaunchKernelGGL((permute_gather_kernel<U_>), grid, block, 0, s, (const uint4*)x, topk_idx, \
                     slot_row, row_token, hist, offsets, (uint4*)x_perm, T, E, k, cap, row_vecs)
  if (row_vecs >= 256) MOE_GATHER(4);   // 4 x 1 KB per chunk keeps the kernel spill-free
  else if (row_vecs >= 128) MOE_GATHER(2);
  else MOE_GATHER(1);
#undef MOE_GATHER
  return hipGetLastError();
}

hipError_t launch_permute_routed(const int32_t* topk_idx, const int32_t* cnt_hist,
                                 int32_t* counts, int32_t* offsets, int32_t* row_token,
                                 int32_t* slot_row, int32_t* perm_flags, int32_t* gen,
                                 int32_t* gen_copy, int T, int E, int k, int cap,
                                 hipStream_t s) {
  if (E > kRoutedExperts || (T + kRouteCountTokens - 1) / kRouteCountTokens > kRoutedMaxBlocks)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(permute_scan_rows_kernel<kRouteCountTokens>, dim3((T + 255) / 256),
                     dim3(256), 0, s, topk_idx, cnt_hist, counts, offsets, row_token, slot_row,
                     perm_flags, gen, gen_copy, nullptr, T, E, k, cap);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// The permutation without a caller workspace, for callers that cannot allocate device
// memory (code under graph capture, tight serving loops): its scratch -- the per-block
// histograms, then the per-block flags -- lives in this file-scope array. Each device that
// runs it holds its own copy until the process ends; every call on a device shares that
// copy, so calls that overlap on one device race. Nothing in it needs to start at zero:
// the count kernel writes every histogram entry and flag word it later reads.
static __device__ __align__(256) int32_t scratch[kNoAllocScratchWords];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int32_t*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

// The device address of `scratch` on the current device, looked up once per device (the
// host-side name of the array is not a device address).
static hipError_t noalloc_scratch(int32_t** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int32_t* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* q = nullptr;
      err = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
      if (err != hipSuccess) return err;
      if (q == nullptr) return hipErrorInvalidSymbol;
      p = static_cast<int32_t*>(q);
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

size_t permute_noalloc_words(int T, int E) {
  return (size_t)permute_count_blocks(T) * ((size_t)E + 1);
}

hipError_t launch_permute_noalloc(const void* x, int elem_bytes, const int32_t* topk_idx,
                                  void* x_perm, int32_t* counts, int32_t* offsets,
                                  int32_t* row_token, int32_t* slot_row, int32_t* flag_out,
                                  int T, int H, int E, int k, int cap, hipStream_t s) {
  if (permute_noalloc_words(T, E) > (size_t)kNoAllocScratchWords) return hipErrorInvalidValue;
  int32_t* base = nullptr;
  const hipError_t err = noalloc_scratch(&base);
  if (err != hipSuccess) return err;
  const int NB = permute_count_blocks(T);
  int32_t* hist = base;                        // [NB][E]
  int32_t* flags = base + (size_t)NB * E;      // [NB]
  return launch_permute(x, elem_bytes, topk_idx, x_perm, counts, offsets, row_token, slot_row,
                        hist, flags, nullptr, nullptr, flag_out, T, H, E, k, cap, s);
}

}  // namespace moe
