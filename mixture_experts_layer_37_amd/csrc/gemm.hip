// Grouped expert GEMMs. Rows of x_perm are grouped by expert (expert e owns rows
// [offsets[e], offsets[e+1])); each expert's rows are multiplied by that expert's weight.
//
// GEMM 1 is the up-projection hidden -> inter with the activation fused into its epilogue
// (lshu.cn/news/82007, section 3: npu_moe_final_optimizer_mm computes the up-projection
// x[tokens,hidden] x W[E,hidden,inter]; activation and down-projection follow). For SwiGLU
// the gate and up projections of the same output columns are computed together, so
// h = silu(x Wg) * (x Wu) never leaves registers. GEMM 2 is the down-projection.
// The pages run one matmul per expert (gitcode.csdn.net MoE page, "核心代码解析": a loop
// over experts); here every expert is one launch, as a persistent grid over a tile list
// that is built on the device from the offsets, so no per-expert sizes reach the host.
//
// gfx950 design (bf16):
//   - block tile 256 x 256 x 64, 4 waves in 2 x 2, each wave 128 x 128 of output computed
//     with v_mfma_f32_32x32x16_bf16 (fp32 accumulators);
//   - A (x_perm rows, K-contiguous) and B (weights [K,N], N-contiguous) are staged through
//     double-buffered LDS (2 x 64 KB); B is transposed in registers (8x8 bf16 blocks) on its
//     way into LDS so that every MFMA operand is one 16-byte K-contiguous LDS read;
//   - LDS rows are 128 B (64 bf16 of K); 16-byte chunks are XOR-swizzled with
//     (row ^ row>>3) & 7, which keeps both the stores and the MFMA reads conflict-free;
//   - operands are issued as (W, x) so each lane's accumulators hold 4 consecutive output
//     columns of one row, written straight to global memory as 8-byte stores;
//   - persistent grid of one block per CU; tiles are ordered (expert, n-tile, m-tile) and
//     each of the 8 XCDs walks its own contiguous range, so the blocks sharing an XCD's L2
//     work on the same weight columns at the same time.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int BM = 256;
constexpr int BK = 64;
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// Per-expert tile starts for tiles of BMt rows x NT column tiles; returns total tiles.
// Uses s_start[0..E] and s_off[0..E] in LDS; 256 threads, E <= 256. Offsets are clamped
// to [0, max_rows] and empty ranges count as empty, so no offsets content can send a tile
// outside the row buffers.
template <int BMt>
__device__ __forceinline__ int build_tile_starts(const int32_t* __restrict__ offsets, int E,
                                                 int NT, int max_rows, int* s_start,
                                                 int* s_off, int* s_wsum) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int tiles = 0;
  for (int i = tid; i <= E; i += blockDim.x) s_off[i] = min(max(offsets[i], 0), max_rows);
  __syncthreads();
  if (tid < E) {
    const int m = max(s_off[tid + 1] - s_off[tid], 0);
    tiles = ((m + BMt - 1) / BMt) * NT;
  }
  int incl = tiles;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(incl, o);
    if (lane >= o) incl += n;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int pre = 0;
  for (int w = 0; w < wave; ++w) pre += s_wsum[w];
  if (tid < E) s_start[tid + 1] = incl + pre;
  if (tid == 0) s_start[0] = 0;
  __syncthreads();
  return s_start[E];
}

// Largest e in [0, E) with s_start[e] <= tile (experts without tiles have equal starts).
__device__ __forceinline__ int find_expert(const int* s_start, int E, int tile) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s_start[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}
__device__ __forceinline__ float gelu_f(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

// Lower/upper 16-bit halves of two words interleaved: element j of rows p and q.
__device__ __forceinline__ uint32_t pair_col(uint32_t p, uint32_t q, int odd) {
  return odd ? ((p >> 16) | (q & 0xffff0000u)) : ((p & 0xffffu) | (q << 16));
}

template <int EPI>
__global__ __launch_bounds__(256, 1) void grouped_gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ offsets,
    const bf16_t* __restrict__ W0, const bf16_t* __restrict__ W1, bf16_t* __restrict__ C, int E,
    int K, int N, int max_rows) {
  constexpr int OUTN = (EPI == EPI_SWIGLU) ? 128 : 256;   // output columns per tile
  __shared__ __attribute__((aligned(16))) bf16_t smem[2][2][BM * BK];
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_wsum[4];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int NT = N / OUTN;
  const int total = build_tile_starts<BM>(offsets, E, NT, max_rows, s_start, s_off, s_wsum);

  const int xcd = blockIdx.x % kXcds, li = blockIdx.x / kXcds;
  const int nper = gridDim.x / kXcds;
  const int per = (total + kXcds - 1) / kXcds;
  const int KT = K / BK;

  // global->LDS staging coordinates
  const int a_c = tid & 7, a_r = tid >> 3;           // A: chunk a_c of rows a_r + 32 i
  const int b_nc = tid & 31, b_kc = tid >> 5;        // B: 8x8 block (n chunk, k chunk)
  // MFMA fragment coordinates
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lhi = lane >> 5;

  for (int it = li; it < per; it += nper) {
    const int tile = xcd * per + it;
    if (tile >= total) break;
    const int e = find_expert(s_start, E, tile);
    const int row_beg = s_off[e];
    const int m_e = s_off[e + 1] - row_beg;   // > 0: the expert owns this tile
    const int mt_e = (m_e + BM - 1) / BM;
    const int rem = tile - s_start[e];
    const int n_t = rem / mt_e, m_t = rem - n_t * mt_e;
    const int row0 = row_beg + m_t * BM;
    const int mrows = min(BM, m_e - m_t * BM);

    // A row offsets (rows past the expert's end re-read its last row; results discarded)
    int a_off[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = min(a_r + 32 * i, mrows - 1);
      a_off[i] = r * K + a_c * 8;
    }
    const bf16_t* Ab = A + (size_t)row0 * K;
    const bf16_t* Bb;
    if (EPI == EPI_SWIGLU) {
      const int col = n_t * 128 + (b_nc & 15) * 8;
      Bb = (b_nc < 16 ? W0 : W1) + (size_t)e * K * N + col;
    } else {
      Bb = W0 + (size_t)e * K * N + n_t * 256 + b_nc * 8;
    }
    Bb += (size_t)(b_kc * 8) * N;

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    uint4 ra[8], rb[8];
    auto gload = [&](int kt) {
      const int k0 = kt * BK;
#pragma unroll
      for (int i = 0; i < 8; ++i) ra[i] = *(const uint4*)(Ab + a_off[i] + k0);
      const bf16_t* bp = Bb + (size_t)k0 * N;
#pragma unroll
      for (int r = 0; r < 8; ++r) rb[r] = *(const uint4*)(bp + (size_t)r * N);
    };
    auto sstore = [&](int buf) {
      bf16_t* As = smem[buf][0];
      bf16_t* Bs = smem[buf][1];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = a_r + 32 * i;
        *(uint4*)(As + r * BK + ((a_c ^ swz(r)) << 3)) = ra[i];
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int n = b_nc * 8 + j;
        const int w = j >> 1, odd = j & 1;
        uint4 o;
        o.x = pair_col((&rb[0].x)[w], (&rb[1].x)[w], odd);
        o.y = pair_col((&rb[2].x)[w], (&rb[3].x)[w], odd);
        o.z = pair_col((&rb[4].x)[w], (&rb[5].x)[w], odd);
        o.w = pair_col((&rb[6].x)[w], (&rb[7].x)[w], odd);
        *(uint4*)(Bs + n * BK + ((b_kc ^ swz(n)) << 3)) = o;
      }
    };
    auto compute = [&](int buf) {
      const bf16_t* As = smem[buf][0];
      const bf16_t* Bs = smem[buf][1];
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int ch = kk * 2 + lhi;
        bf16x8 xa[4], wb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = wm * 128 + i * 32 + l32;
          xa[i] = *(const bf16x8*)(As + m * BK + ((ch ^ swz(m)) << 3));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int nb;
          if (EPI == EPI_SWIGLU) nb = (j < 2 ? 0 : 128) + wn * 64 + (j & 1) * 32;
          else nb = wn * 128 + j * 32;
          const int n = nb + l32;
          wb[j] = *(const bf16x8*)(Bs + n * BK + ((ch ^ swz(n)) << 3));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wb[j], xa[i], acc[i][j], 0, 0, 0);
      }
    };

    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < KT) gload(kt + 1);
      compute(cur);
      if (kt + 1 < KT) sstore(cur ^ 1);
      __syncthreads();
    }

    // Epilogue. acc[i][j][4q+s]: row m = wm*128 + i*32 + l32,
    // column (within the wave's block j) = 8q + 4*lhi + s.
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wm * 128 + i * 32 + l32;
      if (m >= mrows) continue;
      bf16_t* crow = C + (size_t)(row0 + m) * N;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float hv[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
              hv[s] = silu_f(acc[i][j][4 * q + s]) * acc[i][j + 2][4 * q + s];
            const int col = n_t * 128 + wn * 64 + j * 32 + 8 * q + 4 * lhi;
            *(uint2*)(crow + col) = make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
          }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float hv[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const float v = acc[i][j][4 * q + s];
              hv[s] = (EPI == EPI_GELU) ? gelu_f(v) : v;
            }
            const int col = n_t * 256 + wn * 128 + j * 32 + 8 * q + 4 * lhi;
            *(uint2*)(crow + col) = make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
          }
      }
    }
  }
}

static int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  return cus;
}

hipError_t launch_gemm_bf16(int epi, const bf16_t* a, const int32_t* offsets, const bf16_t* w0,
                            const bf16_t* w1, bf16_t* c, int E, int K, int N, int max_rows,
                            hipStream_t s) {
  const int outn = epi == EPI_SWIGLU ? 128 : 256;
  const long max_tiles = (long)((max_rows + BM - 1) / BM + E) * (N / outn);
  int grid = device_cus();
  grid = (grid / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  const long need = ((max_tiles + kXcds - 1) / kXcds) * kXcds;
  if (need < grid) grid = (int)need;
  const dim3 g(grid), b(256);
  switch (epi) {
    case EPI_SWIGLU:
      hipLaunchKernelGGL((grouped_gemm_bf16_kernel<EPI_SWIGLU>), g, b, 0, s, a, offsets, w0, w1, c, E, K, N, max_rows);
      break;
    case EPI_GELU:
      hipLaunchKernelGGL((grouped_gemm_bf16_kernel<EPI_GELU>), g, b, 0, s, a, offsets, w0, w1, c, E, K, N, max_rows);
      break;
    default:
      hipLaunchKernelGGL((grouped_gemm_bf16_kernel<EPI_NONE>), g, b, 0, s, a, offsets, w0, w1, c, E, K, N, max_rows);
      break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// float32 path: plain 16x16 LDS-tiled grouped GEMM on the vector ALUs (for fp32 layers).
constexpr int FT = 16;

template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ offsets, const float* __restrict__ W0,
    const float* __restrict__ W1, float* __restrict__ C, int E, int K, int N, int max_rows) {
  __shared__ float As[FT][FT + 1], B0[FT][FT + 1], B1[FT][FT + 1];
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_wsum[4];
  const int total = build_tile_starts<FT>(offsets, E, 1, max_rows, s_start, s_off, s_wsum);
  const int tile = blockIdx.x;
  if (tile >= total) return;
  const int e = find_expert(s_start, E, tile);
  const int row_beg = s_off[e], m_e = s_off[e + 1] - row_beg;
  const int m_t = tile - s_start[e];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int row = m_t * FT + ty;            // within the expert
  const int col = blockIdx.y * FT + tx;
  const float* We0 = W0 + (size_t)e * K * N;
  const float* We1 = (EPI == EPI_SWIGLU) ? W1 + (size_t)e * K * N : nullptr;
  float acc0 = 0.f, acc1 = 0.f;
  for (int k0 = 0; k0 < K; k0 += FT) {
    const int ka = k0 + tx, kb = k0 + ty;
    As[ty][tx] = (row < m_e && ka < K) ? A[(size_t)(row_beg + row) * K + ka] : 0.f;
    B0[ty][tx] = (kb < K && col < N) ? We0[(size_t)kb * N + col] : 0.f;
    if (EPI == EPI_SWIGLU) B1[ty][tx] = (kb < K && col < N) ? We1[(size_t)kb * N + col] : 0.f;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FT; ++kk) {
      acc0 = fmaf(As[ty][kk], B0[kk][tx], acc0);
      if (EPI == EPI_SWIGLU) acc1 = fmaf(As[ty][kk], B1[kk][tx], acc1);
    }
    __syncthreads();
  }
  if (row < m_e && col < N) {
    float v;
    if (EPI == EPI_SWIGLU) v = (acc0 / (1.0f + expf(-acc0))) * acc1;
    else if (EPI == EPI_GELU) v = 0.5f * acc0 * (1.0f + erff(acc0 * 0.70710678118654752f));
    else v = acc0;
    C[(size_t)(row_beg + row) * N + col] = v;
  }
}

hipError_t launch_gemm_f32(int epi, const float* a, const int32_t* offsets, const float* w0,
                           const float* w1, float* c, int E, int K, int N, int max_rows,
                           hipStream_t s) {
  const dim3 g((max_rows + FT - 1) / FT + E, (N + FT - 1) / FT), b(256);
  switch (epi) {
    case EPI_SWIGLU:
      hipLaunchKernelGGL((grouped_gemm_f32_kernel<EPI_SWIGLU>), g, b, 0, s, a, offsets, w0, w1, c, E, K, N, max_rows);
      break;
    case EPI_GELU:
      hipLaunchKernelGGL((grouped_gemm_f32_kernel<EPI_GELU>), g, b, 0, s, a, offsets, w0, w1, c, E, K, N, max_rows);
      break;
    default:
      hipLaunchKernelGGL((grouped_gemm_f32_kernel<EPI_NONE>), g, b, 0, s, a, offsets, w0, w1, c, E, K, N, max_rows);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
