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
// GEMM 1 can also read its rows straight from the token matrix through the permutation's
// row -> token map, which fuses the permute gather into its operand loads (the pages'
// case for fusing permute with the matmul: lshu.cn/news/82007, section 1).
//
// gfx950 design (bf16):
//   - block tile 256 x 256 x 64, 4 waves in 2 x 2, each wave 128 x 128 of output computed
//     with v_mfma_f32_32x32x16_bf16 (fp32 accumulators in AGPRs);
//   - both operands go global -> LDS by DMA (global_load_lds_dwordx4: lane l's 16 bytes land
//     at base + 16 l), double-buffered in two distinct LDS objects, one barrier per k-step,
//     no register staging. The DMA of step kt + 2 is issued right after the barrier of step
//     kt, under the MFMAs of that step's last k slice;
//   - inside a k-step, each 16-wide k slice first issues the next slice's 12 LDS reads, then
//     runs its 16 MFMAs on fragments read one slice earlier, so LDS latency hides under MFMA
//     execution (fragments double-buffered in VGPRs, accumulators in AGPRs, no spills);
//   - A (x_perm rows, K-contiguous) sits in LDS as [m][64 k], 16-byte chunks XOR-swizzled
//     with (m ^ m>>3) & 7; MFMA fragments are single ds_read_b128;
//   - B (weights [K,N], N-contiguous) stays in its own layout, [64 k][256 n], 32-byte chunks
//     XOR-swizzled with (k & 3) | (k & 1) << 2; MFMA fragments (8 consecutive k of one n
//     per lane) come from two ds_read_b64_tr_b16, the gfx950 transposing LDS read: in each
//     16-lane group lane L reads row L/4, columns 4(L%4)..+3 of a 4 x 16 block and
//     receives column L, rows 0..3. Both swizzles keep reads conflict-free for 32 and 64
//     banks;
//   - operands are issued as (W, x) so each lane's accumulators hold 4 consecutive output
//     columns of one row, written straight to global memory as 8-byte stores (the packed
//     kernel's single-matrix epilogues instead pass the tile through LDS and store whole
//     512-byte rows);
//   - persistent grid of one block per CU; tiles are ordered (expert, n-tile, m-tile) and
//     run round by round: each round of the grid is a contiguous stretch of the list, cut
//     into 8 contiguous pieces, one per XCD. The blocks sharing an XCD's L2 then work on the
//     same weight columns and token rows at the same time, and the XCDs of one round read
//     the rows of the same one or two experts, so a row fetched from HBM by one XCD is found
//     in the Infinity Cache by the others (instead of each XCD streaming its own expert's
//     rows, several times over, from HBM);
//   - split-K tail (GEMM 2, when the caller supplies a partial buffer): the tiles beyond the
//     last whole round of the grid would leave most CUs idle for one full tile time, so each
//     of them is cut into S slices of K (S a power of two, tail * S <= grid), every slice
//     writes a float32 partial tile, and a small reduction kernel adds the S partials in
//     slice order and writes the bf16 rows. The result is deterministic.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "packed_kloop.h"
#include "tile_order.h"

namespace moe {

constexpr int BM = 256;
constexpr int BK = 64;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// The tile order itself (classes, merged order, paired ragged ends) is tile_order.h's.

// Per-expert tile starts in that list; returns the total. s_perm[slot] is the expert in
// list slot `slot`, s_start[slot] its first tile, n_wide the wide experts' tiles (the
// second part starts there). Uses s_start, s_perm, s_off [0..E] and s_wsum[4] in LDS; 256
// threads, E <= 256. Offsets are clamped to [0, max_rows] and empty ranges count as empty,
// so no offsets content can send a tile outside the row buffers. kClasses = false keeps
// every expert in the first part (index order, no merge).
template <int BMt, bool kClasses, bool kPairs = false>
__device__ __forceinline__ int build_tile_starts(const int32_t* __restrict__ offsets, int E,
                                                 int NT, int max_rows, int* s_start,
                                                 int* s_perm, int* s_off, int* s_wsum,
                                                 int& n_wide) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // exclusive scan of v over the block's 256 threads (4 waves)
  auto block_scan = [&](int v, int& total) {
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(incl, o);
      if (lane >= o) incl += n;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int pre = 0;
    for (int w = 0; w < wave; ++w) pre += s_wsum[w];
    total = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    __syncthreads();
    return incl + pre - v;
  };
  for (int i = tid; i <= E; i += blockDim.x) s_off[i] = min(max(offsets[i], 0), max_rows);
  __syncthreads();
  const int m = tid < E ? max(s_off[tid + 1] - s_off[tid], 0) : 0;
  const int small = (kClasses && tid < E && m > 0 && m <= kSmallRows) ? 1 : 0;
  int n_small = 0;
  const int small_before = block_scan(small, n_small);
  if (tid < E) s_perm[small ? (E - n_small) + small_before : tid - small_before] = tid;
  __syncthreads();
  int tiles = 0;
  if (tid < E) {
    const int e = s_perm[tid];
    const int me = max(s_off[e + 1] - s_off[e], 0);
    tiles = expert_tiles(me, NT, BMt, kPairs);
  }
  int total = 0;
  const int before = block_scan(tiles, total);
  if (tid < E) s_start[tid] = before;
  if (tid == 0) s_start[E] = total;
  __syncthreads();
  n_wide = __builtin_amdgcn_readfirstlane(s_start[E - n_small]);   // the small part's start
  return __builtin_amdgcn_readfirstlane(total);
}

// Where a tile sits: its expert, first row, valid rows and n-tile (pair: n-tiles n_t and
// n_t + 1, at most 128 rows).
struct TileCoord {
  int e, row0, mrows, n_t, pair;
};
// The tile at merged position p (NT: n-tiles per m-tile).
template <bool kPairs = false>
__device__ __forceinline__ TileCoord decode_tile(const int* s_start, const int* s_perm,
                                                 const int* s_off, int E, int nw, int total,
                                                 int run, int p, int BMt, int NT) {
  TileCoord t;
  const int tile = merged_tile(p, nw, total, run);
  const int slot = find_expert(s_start, E, tile);
  t.e = s_perm[slot];
  const int row_beg = s_off[t.e];
  const int m_e = s_off[t.e + 1] - row_beg;   // > 0: the expert owns this tile
  const TileInExpert te = tile_in_expert(m_e, tile - s_start[slot], NT, BMt, kPairs);
  t.n_t = te.n_t;
  t.pair = te.pair;
  const int m_t = te.m_t;
  t.row0 = row_beg + m_t * BMt;
  t.mrows = min(BMt, m_e - m_t * BMt);
  return t;
}

// Split-K plan of one launch: tiles [0, full) run whole, tiles [full, full + tail) run as
// S slices of K each (S = 1: no split, full = total). Slices are whole pairs of k-steps, at
// least 16 k-steps long, and tail * S fits both the grid and the partial buffer.
struct SplitPlan {
  int full, tail, S;
};
constexpr int kMaxSplit = 8;
__device__ __forceinline__ SplitPlan split_plan(int total, int grid, int KT, bool enabled) {
  SplitPlan p = {total, 0, 1};
  if (!enabled) return p;
  const int full = (total / grid) * grid, tail = total - full;
  const int units = min(grid, kSplitMaxUnits);
  int S = 1;
  while (tail > 0 && S < kMaxSplit && tail * S * 2 <= units && KT >= 16 * S * 2) S *= 2;
  if (S > 1) {
    p.full = full;
    p.tail = tail;
    p.S = S;
  }
  return p;
}
// k-steps [kb, ke) of slice c of S (KT even).
__device__ __forceinline__ void slice_range(int KT, int S, int c, int& kb, int& ke) {
  const int pairs = KT / 2;
  kb = 2 * (c * pairs / S);
  ke = 2 * ((c + 1) * pairs / S);
}

__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}
__device__ __forceinline__ float gelu_f(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}
// d/dz of z Phi(z) = Phi(z) + z phi(z)
__device__ __forceinline__ float gelu_grad_f(float z) {
  return 0.5f * (1.0f + erff(z * 0.70710678118654752f)) +
         z * 0.39894228040143268f * __expf(-0.5f * z * z);
}
// four floats <-> four packed bf16 (8 bytes)
__device__ __forceinline__ uint2 pack4(const float* v) {
  return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
__device__ __forceinline__ void unpack4(uint2 w, float* v) {
  v[0] = bf16_to_f32(w.x & 0xffffu);
  v[1] = bf16_to_f32(w.x >> 16);
  v[2] = bf16_to_f32(w.y & 0xffffu);
  v[3] = bf16_to_f32(w.y >> 16);
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef short v8i16 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// B-tile swizzle of 32-byte chunks for row k (a row is 128 columns = 256 bytes).
__device__ __forceinline__ int bswz(int k) { return (k & 3) | ((k & 1) << 2); }

// 16 bytes per lane global -> LDS: lane l's bytes land at lds + 16 l (lds is wave-uniform).
__device__ __forceinline__ void lds_dma16(const void* src, bf16_t* lds) {
  __builtin_amdgcn_global_load_lds((global_void*)src, (lds_void*)lds, 16, 0, 0);
}

// MFMA operand fragments of one 16-wide k slice of a wave's 128 x 128 output block.
struct Frags {
  bf16x8 a[4];   // token rows   wm*128 + 32 i + (lane & 31)
  bf16x8 b[4];   // weight columns of the wave's four 32-column blocks
};

constexpr int kHalf = BK * 128;                  // elements of one B half [64 k][128 n]
constexpr int kStage = BM * BK + 2 * kHalf;      // elements of one LDS stage (64 KB)

// A rows: row r of the expert-major operand is A[r] (row_token == nullptr) or, with the
// permute gather fused in, token row A[row_token[r]] (clamped into [0, a_rows)).
template <int EPI, bool BT>
__global__ __launch_bounds__(256, 1) void grouped_gemm_bf16_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ row_token, int a_rows,
    const int32_t* __restrict__ offsets, const bf16_t* __restrict__ W0,
    const bf16_t* __restrict__ W1, bf16_t* __restrict__ C, float* __restrict__ partial,
    const bf16_t* __restrict__ aux, const int32_t* __restrict__ aux_off,
    bf16_t* __restrict__ C2, int E, int K, int N, int max_rows) {
  // Two stages in two distinct LDS objects: the compiler can then tell a DMA into one
  // stage from reads of the other and does not make those reads wait for the DMA.
  __shared__ __attribute__((aligned(1024))) bf16_t stage0[kStage];
  __shared__ __attribute__((aligned(1024))) bf16_t stage1[kStage];
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_perm[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_wsum[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Two-matrix tiles (gate and up columns of the same outputs) or one matrix of 256 columns.
  constexpr bool kTwoMat = (EPI == EPI_SWIGLU || EPI == EPI_GU);
  static_assert(!(BT && kTwoMat), "transposed weights: single-matrix epilogues only");
  constexpr int OUTN = kTwoMat ? 128 : 256;   // output columns per tile
  // Row strides of C and of the epilogue's second input (aux): the gate/up pair buffers
  // [rows, 2N] hold the gate half in columns [0, N) and the up half in [N, 2N).
  constexpr bool kPairOut = (EPI == EPI_GU || EPI == EPI_SWIGLU_BWD);
  const size_t ldc = kPairOut ? 2 * (size_t)N : (size_t)N;
  const size_t ldaux = (EPI == EPI_SWIGLU_BWD) ? 2 * (size_t)N : (size_t)N;
  const int NT = N / OUTN;
  int n_wide = 0;
  const int total =
      build_tile_starts<BM, true>(offsets, E, NT, max_rows, s_start, s_perm, s_off, s_wsum, n_wide);

  const int xcd = blockIdx.x % kXcds, li = blockIdx.x / kXcds;
  const int nper = gridDim.x / kXcds;
  const int KT = K / BK;
  const SplitPlan plan = split_plan(__builtin_amdgcn_readfirstlane(total), gridDim.x, KT,
                                   EPI == EPI_NONE && partial != nullptr);
  const int my_unit = xcd * nper + li;                // this block's split slice, if any

  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lhi = lane >> 5;

  // Per-lane LDS read offsets (bytes within a stage). A fragment (kk, i): row
  // m = wm*128 + 32 i + l32, 16-byte chunk 2 kk + lhi, stored at chunk ^ swz(m); swz
  // changes only in bit 2 with i & 1, applied as an XOR below.
  uint32_t a_rd[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int m = wm * 128 + l32;
    a_rd[kk] = (uint32_t)(m * BK * 2 + (((kk * 2 + lhi) ^ swz(m)) << 4));
  }
  // B fragment (kk, j): 8 consecutive k of one weight column per lane from two
  // ds_read_b64_tr_b16 (rows krow0 + 16 kk and krow0 + 16 kk + 4). The swizzle depends on
  // k & 3 only, so kk is an immediate offset.
  // With BT (weights given transposed, [N][K] with K contiguous) B sits in LDS like A,
  // [256 n][64 k] swizzled, and its fragments are single ds_read_b128 as well.
  uint32_t b_rd_bt[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int n = wn * 128 + l32;
    b_rd_bt[kk] = (uint32_t)((BM * BK + n * BK) * 2 + (((kk * 2 + lhi) ^ swz(n)) << 4));
  }
  uint32_t b_rd[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int h, nb;
    if (kTwoMat) { h = j >> 1; nb = wn * 64 + (j & 1) * 32; }
    else { h = wn; nb = j * 32; }
    const int krow0 = 8 * lhi + ((lane & 15) >> 2);
    const int c32 = (nb >> 4) + ((lane >> 4) & 1);
    b_rd[j] = (uint32_t)((BM * BK + h * kHalf) * 2 + krow0 * 256 + ((c32 ^ bswz(krow0)) << 5) +
                         8 * (lane & 3));
  }

  auto load_frags = [&](const bf16_t* stg, int kk, Frags& f) {
    const char* st = (const char*)stg;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = a_rd[kk] ^ ((i & 1) << 6);
      f.a[i] = *(const bf16x8*)(st + off + i * 32 * BK * 2);
    }
    if constexpr (BT) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t off = b_rd_bt[kk] ^ ((j & 1) << 6);
        f.b[j] = *(const bf16x8*)(st + off + j * 32 * BK * 2);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const char* p = st + b_rd[j] + kk * 16 * 256;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const lds_char*)p);
        const v4i16 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const lds_char*)(p + 4 * 256));
        const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        f.b[j] = __builtin_bit_cast(bf16x8, v);
      }
    }
  };

  // One work item: tile `tile`, k-steps [kb, ke). A slice item (GEMM 2's split-K tail)
  // writes a float32 partial tile instead of bf16 rows. Each kind has its own call site, so
  // each gets its own register allocation.
  auto run_tile = [&](int tile, int kb, int ke, float* part, auto slice) {
    constexpr bool kSlice = decltype(slice)::value;
    const TileCoord tc = decode_tile(s_start, s_perm, s_off, E, n_wide, total, nper,
                                      __builtin_amdgcn_readfirstlane(tile), BM, NT);
    const int e = __builtin_amdgcn_readfirstlane(tc.e);
    const int n_t = __builtin_amdgcn_readfirstlane(tc.n_t);
    const int row0 = __builtin_amdgcn_readfirstlane(tc.row0);
    const int mrows = __builtin_amdgcn_readfirstlane(tc.mrows);
    // B halves: base pointers (uniform) of columns [0,128) and [128,256) of the tile
    const bf16_t* Bh0;
    const bf16_t* Bh1;
    if (kTwoMat) {
      Bh0 = W0 + (size_t)e * K * N + n_t * 128;
      Bh1 = W1 + (size_t)e * K * N + n_t * 128;
    } else {
      Bh0 = W0 + (size_t)e * K * N + n_t * 256;
      Bh1 = Bh0 + 128;
    }

    // DMA sources of this lane at k0 = 0 (A) / offsets relative to the B halves.
    // A: instruction i of wave w fills chunks [(w*8+i)*64, +64) of [256 m][8 chunks];
    // rows past the expert's last row re-read its last row (never written back).
    const char* a_src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wave * 64 + i * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      const int rr = row0 + min(r, mrows - 1);
      const size_t arow = row_token != nullptr ? (size_t)min(max(row_token[rr], 0), a_rows - 1)
                                               : (size_t)rr;
      a_src[i] = (const char*)(A + arow * K) + c * 16;
    }
    // B: instruction i of wave w fills units [(w*4 + i)*64, +64) of one half's
    // [64 k][16 units]: row k = (w*4 + i)*4 + lane/16.
    uint32_t b_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = (wave * 4 + i) * 4 + (lane >> 4);
      const int u = lane & 15;
      const int ncol = (((u >> 1) ^ bswz(k)) << 4) + ((u & 1) << 3);
      b_src[i] = (uint32_t)(k * N * 2 + ncol * 2);
    }
    // BT: B^T rows n of this tile, K-contiguous, in one or two K parts (W0 for k < Ks,
    // W1 for k >= Ks; each [E][N][Ks]); sources like A's, as byte offsets.
    const int Ks = (BT && W1 != nullptr) ? K / 2 : K;
    uint32_t bt_src[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wave * 64 + i * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      bt_src[i] = (uint32_t)((n_t * 256 + r) * Ks * 2 + c * 16);
    }
    const char* Bt0 = (const char*)(W0 + (size_t)e * N * Ks);
    const char* Bt1 = BT && W1 != nullptr ? (const char*)(W1 + (size_t)e * N * Ks) : Bt0;

    auto dma = [&](int kt, bf16_t* stg) {
      const uint32_t kA = (uint32_t)(kt * BK * 2);
      const size_t kB = (size_t)kt * BK * N * 2;
#pragma unroll
      for (int i = 0; i < 8; ++i) lds_dma16(a_src[i] + kA, stg + (wave * 8 + i) * 512);
      if constexpr (BT) {
        const int k0 = kt * BK;
        const char* bb = k0 < Ks ? Bt0 + k0 * 2 : Bt1 + (k0 - Ks) * 2;
#pragma unroll
        for (int i = 0; i < 8; ++i) lds_dma16(bb + bt_src[i], stg + BM * BK + (wave * 8 + i) * 512);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          lds_dma16((const char*)Bh0 + kB + b_src[i], stg + BM * BK + (wave * 4 + i) * 512);
          lds_dma16((const char*)Bh1 + kB + b_src[i],
                    stg + BM * BK + kHalf + (wave * 4 + i) * 512);
        }
      }
    };

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    auto mfma16 = [&](const Frags& f) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
    };
    // One 16-wide k slice: the next slice's 12 LDS reads go out first, then the 16 MFMAs
    // of the current slice run while they are in flight. The reads issued one slice earlier
    // are drained first (they have had a whole slice to land): the 4-bit LDS counter cannot
    // track 24 outstanding reads, and without this wait the compiler waits for all of them
    // after issuing the new ones.
    auto phase = [&](const bf16_t* stg, int kk_next, Frags& nxt, const Frags& cur) {
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0Only);
      load_frags(stg, kk_next, nxt);
      mfma16(cur);
      __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);   // the LDS reads
      __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);   // then the MFMAs
      __builtin_amdgcn_sched_barrier(0);
    };
    Frags f0, f1;
    // One k-step on stage `cur` while stage `nxt` is in flight. After its last LDS read of
    // `cur`, the wave waits for its own DMA into `nxt`; the barrier then publishes `nxt`
    // and frees `cur`, which is refilled with step kt + 2 under the last slice's MFMAs.
    // `refill` / `next` are compile-time at every call site: the steady-state loop carries
    // no branches, which keeps the fragments in VGPRs and the accumulators in AGPRs.
    auto kstep = [&](int kt, bf16_t* cur, bf16_t* nxt, auto refill, auto next) {
      phase(cur, 1, f1, f0);
      phase(cur, 2, f0, f1);
      phase(cur, 3, f1, f0);
      __builtin_amdgcn_s_waitcnt(0);   // f1 has landed; this wave's DMA into nxt is done
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(refill)::value) dma(kt + 2, cur);
      if constexpr (decltype(next)::value) load_frags(nxt, 0, f0);
      mfma16(f1);
      __builtin_amdgcn_sched_barrier(0);
    };
    using yes = std::true_type;
    using no = std::false_type;

    // ke - kb is even (K is a multiple of 128 and slices are whole pairs), so the steps
    // pair up as (stage0, stage1).
    dma(kb, stage0);
    __builtin_amdgcn_s_waitcnt(0);
    dma(kb + 1, stage1);
    __syncthreads();
    load_frags(stage0, 0, f0);
    int kt = kb;
    for (; kt + 2 < ke; kt += 2) {
      kstep(kt, stage0, stage1, yes{}, yes{});
      kstep(kt + 1, stage1, stage0, yes{}, yes{});
    }
    kstep(kt, stage0, stage1, no{}, yes{});
    kstep(kt + 1, stage1, stage0, no{}, no{});
    __syncthreads();   // every wave is done with both stages before the next tile's DMA

    // Epilogue. acc[i][j][4q+s]: row m = wm*128 + i*32 + l32,
    // column (within the wave's block j) = 8q + 4*lhi + s.
    if constexpr (kSlice) {   // float32 partial tile [BM][256], valid rows only
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = wm * 128 + i * 32 + l32;
        if (m >= mrows) continue;
        float* prow = part + (size_t)m * 256;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = wn * 128 + j * 32 + 8 * q + 4 * lhi;
            *(float4*)(prow + col) = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                 acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          }
      }
      return;
    }
    if constexpr (EPI == EPI_SWIGLU_BWD) {
      // The float32 dh tile leaves through LDS (the two stages, free after the barrier
      // above), 64 rows at a time, and is read back in row order: each lane then loads the
      // saved g and u and stores dg and du as 16-byte pieces of whole 512-byte row segments,
      // instead of 8-byte pieces scattered over 32 rows per instruction. 16-byte chunk c of
      // LDS row r (1 KB) sits at c ^ (r & 31). LDS-only barriers.
      constexpr int kRowB = 1024;
      // Tile coordinates and lane index pass through empty asm, so no address below is
      // computed (and held in registers) across the k-loop.
      int e_row0 = row0, e_nt = n_t, e_mrows = mrows, e_e = e, e_lane = lane, e_tid = tid;
      asm volatile("" : "+s"(e_row0), "+s"(e_nt), "+s"(e_mrows), "+s"(e_e));
      asm volatile("" : "+v"(e_lane), "+v"(e_tid));
      // aux rows: the C rows themselves, or (aux_off given) the compact rows of a layout
      // without padding: row r of expert e maps to r - offsets[e] + aux_off[e], and pad rows
      // to the expert's last row (their dh is zero)
      int a_lo = 0, a_hi = 0;
      if (aux_off != nullptr) {
        a_lo = aux_off[e_e];
        a_hi = aux_off[e_e + 1];
      }
      const int e_first = s_off[e_e];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        char* buf = (char*)((i & 1) ? stage1 : stage0);
        const int lr = wm * 32 + (e_lane & 31);   // row of this lane's outputs in the block
        const int lh = e_lane >> 5;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int chunk = wn * 32 + j * 8 + 2 * q + lh;   // columns 4 chunk .. 4 chunk + 3
            *(float4*)(buf + lr * kRowB + ((chunk ^ (lr & 31)) << 4)) =
                make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                            acc[i][j][4 * q + 3]);
          }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int gi = r * 256 + e_tid;   // 8-column group of the 64 x 256 block
          const int row = gi >> 5, cg = gi & 31;
          const int m = (row < 32 ? 0 : 128) + i * 32 + (row & 31);
          if (m >= e_mrows) continue;
          const char* lrow = buf + row * kRowB;
          const float4 d0 = *(const float4*)(lrow + (((2 * cg) ^ (row & 31)) << 4));
          const float4 d1 = *(const float4*)(lrow + (((2 * cg + 1) ^ (row & 31)) << 4));
          size_t ar = (size_t)(e_row0 + m);
          if (aux_off != nullptr) ar = (size_t)max(min(e_row0 + m - e_first + a_lo, a_hi - 1), a_lo);
          const bf16_t* arow = aux + ar * ldaux + e_nt * 256 + cg * 8;
          const uint4 gw = *(const uint4*)arow;
          const uint4 uw = *(const uint4*)(arow + N);
          const float dh[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
          float g[8], u[8], dg[8], du[8];
          unpack4(make_uint2(gw.x, gw.y), g);
          unpack4(make_uint2(gw.z, gw.w), g + 4);
          unpack4(make_uint2(uw.x, uw.y), u);
          unpack4(make_uint2(uw.z, uw.w), u + 4);
          // dg = dh u silu'(g), du = dh silu(g)
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-g[s]));
            dg[s] = dh[s] * u[s] * (sg * (1.0f + g[s] * (1.0f - sg)));
            du[s] = dh[s] * g[s] * sg;
          }
          bf16_t* crow = C + (size_t)(e_row0 + m) * ldc + e_nt * 256 + cg * 8;
          const uint2 dg0 = pack4(dg), dg1 = pack4(dg + 4);
          const uint2 du0 = pack4(du), du1 = pack4(du + 4);
          *(uint4*)crow = make_uint4(dg0.x, dg0.y, dg1.x, dg1.y);
          *(uint4*)(crow + N) = make_uint4(du0.x, du0.y, du1.x, du1.y);
        }
      }
      // every wave is done reading the stages before the next tile's DMA refills them
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = wm * 128 + i * 32 + l32;
      if (m >= mrows) continue;
      bf16_t* crow = C + (size_t)(row0 + m) * ldc;
      if constexpr (kTwoMat) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = n_t * 128 + wn * 64 + j * 32 + 8 * q + 4 * lhi;
            if constexpr (EPI == EPI_SWIGLU) {
              float hv[4];
#pragma unroll
              for (int s = 0; s < 4; ++s)
                hv[s] = silu_f(acc[i][j][4 * q + s]) * acc[i][j + 2][4 * q + s];
              *(uint2*)(crow + col) = pack4(hv);
            } else {   // EPI_GU: the gate and up pre-activations, and h into C2
              float gv[4], uv[4], hv[4];
#pragma unroll
              for (int s = 0; s < 4; ++s) {
                gv[s] = acc[i][j][4 * q + s];
                uv[s] = acc[i][j + 2][4 * q + s];
                hv[s] = silu_f(gv[s]) * uv[s];
              }
              *(uint2*)(crow + col) = pack4(gv);
              *(uint2*)(crow + N + col) = pack4(uv);
              *(uint2*)(C2 + (size_t)(row0 + m) * N + col) = pack4(hv);
            }
          }
      } else {
        // aux rows: the C rows themselves, or (aux_off given) the compact rows of a layout
        // without padding: row r of expert e maps to r - offsets[e] + aux_off[e], and pad
        // rows to the expert's last row (their dh is zero)
        size_t ar = (size_t)(row0 + m);
        if (aux_off != nullptr) {
          const int lo = aux_off[e], hi = aux_off[e + 1];
          ar = (size_t)max(min(row0 + m - s_off[e] + lo, hi - 1), lo);
        }
        const bf16_t* arow = aux + ar * ldaux;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = n_t * 256 + wn * 128 + j * 32 + 8 * q + 4 * lhi;
            float hv[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) hv[s] = acc[i][j][4 * q + s];
            if constexpr (EPI == EPI_GELU) {
#pragma unroll
              for (int s = 0; s < 4; ++s) hv[s] = gelu_f(hv[s]);
            } else if constexpr (EPI == EPI_AH) {   // a into C, gelu(a) into C2
              float gv[4];
#pragma unroll
              for (int s = 0; s < 4; ++s) gv[s] = gelu_f(hv[s]);
              *(uint2*)(C2 + (size_t)(row0 + m) * N + col) = pack4(gv);
            } else if constexpr (EPI == EPI_GELU_BWD) {
              // hv = dh; with a the saved pre-activation: da = dh gelu'(a)
              float a[4];
              unpack4(*(const uint2*)(arow + col), a);
#pragma unroll
              for (int s = 0; s < 4; ++s) hv[s] *= gelu_grad_f(a[s]);

            }
            *(uint2*)(crow + col) = pack4(hv);
          }
      }
    }
  };

  // Whole tiles round by round, then at most one split slice per block. Round r covers
  // tiles [r G, (r + 1) G) of the list; XCD x takes the x-th eighth of it, one tile per
  // block.
  for (int base = 0; base < plan.full; base += gridDim.x) {
    const int tile = base + xcd * nper + li;
    if (tile >= plan.full) break;
    run_tile(tile, 0, KT, nullptr, std::false_type{});
  }
  if constexpr (EPI == EPI_NONE) {
    if (my_unit < plan.tail * plan.S) {
      int kb, ke;
      slice_range(KT, plan.S, my_unit % plan.S, kb, ke);
      run_tile(plan.full + my_unit / plan.S, kb, ke, partial + (size_t)my_unit * (BM * 256),
               std::true_type{});
    }
  }
}

int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return 256;
  return cus;
}

// Split-K tail reduction of GEMM 2: for each sliced tile, C rows = bf16(sum over slices, in
// slice order, of the float32 partials). Re-derives the launch's tile list and split plan
// from the same offsets and grid size. Block work item: 8 rows of one tile, 32 threads per
// row, 8 columns per thread.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            const int32_t* __restrict__ offsets,
                                                            bf16_t* __restrict__ C, int E, int K,
                                                            int N, int max_rows, int grid) {
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_perm[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_wsum[4];
  int n_wide = 0;
  const int total = build_tile_starts<BM, true>(offsets, E, N / 256, max_rows, s_start, s_perm,
                                                s_off, s_wsum, n_wide);
  const SplitPlan plan = split_plan(total, grid, K / BK, true);
  const int tid = threadIdx.x;
  for (int w = blockIdx.x; w < plan.tail * (BM / 8); w += gridDim.x) {
    const int ti = w / (BM / 8);
    const TileCoord tc = decode_tile(s_start, s_perm, s_off, E, n_wide, total, grid / kXcds,
                                      plan.full + ti, BM, N / 256);
    const int r = (w % (BM / 8)) * 8 + (tid >> 5);
    if (r >= tc.mrows) continue;
    const int c8 = (tid & 31) * 8;
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int sl = 0; sl < plan.S; ++sl) {
      const float* p = partial + ((size_t)(ti * plan.S + sl) * BM + r) * 256 + c8;
      const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
      acc[0] += a.x; acc[1] += a.y; acc[2] += a.z; acc[3] += a.w;
      acc[4] += b.x; acc[5] += b.y; acc[6] += b.z; acc[7] += b.w;
    }
    *(uint4*)(C + (size_t)(tc.row0 + r) * N + tc.n_t * 256 + c8) =
        make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

hipError_t launch_gemm_bf16(int epi, const bf16_t* a, const int32_t* row_token, int a_rows,
                            const int32_t* offsets, const bf16_t* w0, const bf16_t* w1,
                            bf16_t* c, float* partial, const bf16_t* aux, bf16_t* c2, int E,
                            int K, int N, int max_rows, hipStream_t s) {
  const int outn = (epi == EPI_SWIGLU || epi == EPI_GU) ? 128 : 256;
  const bool split = epi == EPI_NONE && partial != nullptr;
  const long max_tiles = (long)((max_rows + BM - 1) / BM + E) * (N / outn);
  int grid = device_cus();
  grid = (grid / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  // Without a split, no more blocks than tiles; with one, the whole grid (a short tile list
  // is then cut into K slices over all CUs).
  const long need = ((max_tiles + kXcds - 1) / kXcds) * kXcds;
  if (!split && need < grid) grid = (int)need;
  if (!split) partial = nullptr;
  const dim3 g(grid), b(256);
#define MOE_GEMM(EP)                                                                        \
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<EP, false>), g, b, 0, s, a, row_token, a_rows, \
                     offsets, w0, w1, c, partial, aux, nullptr, c2, E, K, N, max_rows)
  switch (epi) {
    case EPI_SWIGLU: MOE_GEMM(EPI_SWIGLU); break;
    case EPI_GELU: MOE_GEMM(EPI_GELU); break;
    case EPI_GU: MOE_GEMM(EPI_GU); break;
    case EPI_SWIGLU_BWD: MOE_GEMM(EPI_SWIGLU_BWD); break;
    case EPI_GELU_BWD: MOE_GEMM(EPI_GELU_BWD); break;
    case EPI_AH: MOE_GEMM(EPI_AH); break;
    default: MOE_GEMM(EPI_NONE); break;
  }
#undef MOE_GEMM
  if (split) {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(1024), dim3(256), 0, s, partial, offsets, c, E,
                       K, N, max_rows, grid);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_bt(int epi, const bf16_t* a, const int32_t* offsets,
                               const bf16_t* w0, const bf16_t* w1, bf16_t* c, float* partial,
                               const bf16_t* aux, const int32_t* aux_off, int E, int K, int N,
                               int max_rows, hipStream_t s) {
  const bool split = epi == EPI_NONE && partial != nullptr;
  const long max_tiles = (long)((max_rows + BM - 1) / BM + E) * (N / 256);
  int grid = device_cus();
  grid = (grid / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  const long need = ((max_tiles + kXcds - 1) / kXcds) * kXcds;
  if (!split && need < grid) grid = (int)need;
  if (!split) partial = nullptr;
  const dim3 g(grid), b(256);
#define MOE_GEMM_BT(EP)                                                                        \
  hipLaunchKernelGGL((grouped_gemm_bf16_kernel<EP, true>), g, b, 0, s, a, nullptr, max_rows,    \
                     offsets, w0, w1, c, partial, aux, aux_off, nullptr, E, K, N, max_rows)
  switch (epi) {
    case EPI_SWIGLU_BWD: MOE_GEMM_BT(EPI_SWIGLU_BWD); break;
    case EPI_GELU_BWD: MOE_GEMM_BT(EPI_GELU_BWD); break;
    case EPI_NONE: MOE_GEMM_BT(EPI_NONE); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_GEMM_BT
  if (split) {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(1024), dim3(256), 0, s, partial, offsets, c, E,
                       K, N, max_rows, grid);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Packed weights. Inference weights are constant, so they can be stored once in the order
// the MFMAs consume them: a bf16 matrix W[E][K][N] packed by pack_weight_kernel holds, for
// expert e, 32-column block nb and 16-row k slice ks, one 1 KB block
//   P[e][nb][ks][l][q] = W[e][16 ks + 8 (l >> 5) + q][32 nb + (l & 31)],  l < 64, q < 8,
// which is exactly lane l's operand of v_mfma_f32_32x32x16_bf16 for those 32 columns and
// 16 k. The packed GEMM then loads each wave's weight fragments straight into registers,
// one coalesced 16-byte load per lane and block, and only the token rows go through LDS:
// per k-step a block moves 32 KB into LDS and reads 64 KB of fragments out of it, against
// 64 KB and 128 KB when both operands are staged. Sums run in the same order as in
// grouped_gemm_bf16_kernel, so the results are bit-identical to it.
__global__ __launch_bounds__(256) void pack_weight_kernel(const bf16_t* __restrict__ W,
                                                          bf16_t* __restrict__ P, int E, int K,
                                                          int N) {
  const int NB = N / 32, KS = K / 16;
  const size_t total = (size_t)E * NB * KS * 64;   // 16-byte chunks of P
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (size_t)gridDim.x * blockDim.x) {
    const int l = (int)(i & 63);
    size_t t = i >> 6;
    const int ks = (int)(t % KS);
    t /= KS;
    const int nb = (int)(t % NB);
    const int e = (int)(t / NB);
    const bf16_t* src = W + ((size_t)e * K + ks * 16 + 8 * (l >> 5)) * N + nb * 32 + (l & 31);
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (uint32_t)src[(size_t)(2 * q) * N] | ((uint32_t)src[(size_t)(2 * q + 1) * N] << 16);
    *(uint4*)(P + i * 8) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Grouped GEMM on packed weights: SWIGLU (P0 gate, P1 up), GELU and NONE (P0), with the
// tile list, round-by-round order, fused gather and split-K tail of
// grouped_gemm_bf16_kernel. Wave wn computes all 256 rows of the tile and two 32-column
// blocks j: SwiGLU gate (j = 0) and up (j = 1) of output columns wn*32 .. +31, else columns
// wn*64 + 32 j. The k-loop (token rows by LDS DMA, weight fragments straight into
// registers, waits derived from its issue order at compile time) is packed_kloop.
template <int EPI>
__global__ __launch_bounds__(256, 1) void grouped_gemm_packed_kernel(
    const bf16_t* __restrict__ A, const int32_t* __restrict__ row_token, int a_rows,
    const int32_t* __restrict__ offsets, const bf16_t* __restrict__ P0,
    const bf16_t* __restrict__ P1, bf16_t* __restrict__ C, float* __restrict__ partial, int E,
    int K, int N, int max_rows) {
  static_assert(EPI == EPI_SWIGLU || EPI == EPI_GELU || EPI == EPI_NONE, "packed epilogues");
  __shared__ __attribute__((aligned(1024))) bf16_t sa0[BM * BK];
  __shared__ __attribute__((aligned(1024))) bf16_t sa1[BM * BK];
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_perm[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_wsum[4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr bool kTwoMat = EPI == EPI_SWIGLU;
  constexpr bool kPairs = EPI == EPI_SWIGLU;   // paired ragged ends (no split-K here)
  constexpr int OUTN = kTwoMat ? 128 : 256;
  const int NT = N / OUTN, NB = N / 32, KS = K / 16;
  int n_wide = 0;
  const int total = build_tile_starts<BM, true, kPairs>(offsets, E, NT, max_rows, s_start, s_perm,
                                                        s_off, s_wsum, n_wide);
  const int xcd = blockIdx.x % kXcds, li = blockIdx.x / kXcds;
  const int nper = gridDim.x / kXcds;
  const int KT = K / BK;
  const SplitPlan plan = split_plan(__builtin_amdgcn_readfirstlane(total), gridDim.x, KT,
                                   EPI == EPI_NONE && partial != nullptr);
  const int my_unit = xcd * nper + li;
  // Wave layout 1 x 4: wave wn owns all 256 rows and 64 columns of the tile, so per slice
  // it reads 8 A fragments from LDS and loads 2 weight fragments, and no weight block is
  // loaded twice per block (a 2 x 2 layout, 128 x 128 per wave, loads each weight block in
  // two waves: a third more cache-line lookups per k-step, measured 1.5-4% slower).
  constexpr int kNA = 8, kNB = 2;
  const int wn = wave;
  const int l32 = lane & 31, lhi = lane >> 5;
  uint32_t a_rd[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) a_rd[kk] = (uint32_t)(l32 * BK * 2 + (((kk * 2 + lhi) ^ swz(l32)) << 4));
  // the first NA (8 or 4) A fragments of slice kk from an LDS stage
  auto load_a = [&](const bf16_t* stg, int kk, auto& f) {
    constexpr int NA = sizeof(f.a) / sizeof(f.a[0]);
    const char* st = (const char*)stg;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const uint32_t off = a_rd[kk] ^ ((i & 1) << 6);
      f.a[i] = *(const bf16x8*)(st + off + i * 32 * BK * 2);
    }
  };

  // Where a tile's operands come from: token rows (A, global -> LDS by DMA; with the gather
  // fused in, rows of x through row_token) and packed weight blocks (B, into registers).
  struct TileSrc {
    int n_t, row0, mrows;
    const char* a_src[8];
    const bf16_t* bsrc[2 * kNB];   // a pair tile: both n-tiles' fragments
  };
  // A tile's coordinates and the token rows of its A DMA loads (8, 4 or 2 per wave by row
  // class; rows past the expert's end re-read its last row, never written back; with the
  // gather fused in, rows of x through row_token, clamped into [0, a_rows)). The row-map
  // loads are the only global loads here.
  // Row classes: full height (8 A fragments); half (4) and quarter (2) height for a tile
  // whose rows are all of an expert of at most 128 and 64 rows (and, with paired ragged
  // ends, for the ragged end of an odd last n-tile); a pair tile (4 A fragments by both
  // n-tiles' weight fragments), and in an expert of at most 64 rows a quarter-height pair
  // tile (2 A fragments by both n-tiles' weight fragments).
  enum { kFull = 0, kHalfRows = 1, kQuarterRows = 2, kPairTile = 3, kPairQuarter = 4 };
  // A DMA loads per k-step and wave of a class: its 32 NA rows, 8 per load, over 4 waves
  // (rows past the expert's end are not loaded for a tile of fewer A fragments)
  auto a_loads = [](int cls) {
    return cls == kFull ? 8 : (cls == kQuarterRows || cls == kPairQuarter) ? 2 : 4;
  };
  struct TileRows {
    int e, n_t, row0, mrows;
    int cls, la;
    int arow[8];
  };
  auto tile_rows = [&](int tile, TileRows& r) {
    // the lane index passes through empty asm, so the per-lane pieces below are computed
    // for each tile rather than hoisted and held across the k-loop
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    const TileCoord tc = decode_tile<kPairs>(s_start, s_perm, s_off, E, n_wide, total, nper,
                                              __builtin_amdgcn_readfirstlane(tile), BM, NT);
    r.e = __builtin_amdgcn_readfirstlane(tc.e);
    r.n_t = __builtin_amdgcn_readfirstlane(tc.n_t);
    r.row0 = __builtin_amdgcn_readfirstlane(tc.row0);
    r.mrows = __builtin_amdgcn_readfirstlane(tc.mrows);
    const int rows_e = __builtin_amdgcn_readfirstlane(s_off[r.e + 1] - s_off[r.e]);
    // the rows that decide the height: the expert's if it has a single m-tile; with paired
    // ragged ends, the tile's (the ragged end of an odd last n-tile)
    const int hrows = (kPairs && rows_e > kSmallRows) ? r.mrows : rows_e;
    r.cls = (kPairs && tc.pair) ? (rows_e <= 64 ? kPairQuarter : kPairTile)
            : hrows <= 64       ? kQuarterRows
            : hrows <= 128      ? kHalfRows
                                : kFull;
    r.cls = __builtin_amdgcn_readfirstlane(r.cls);
    r.la = a_loads(r.cls);
    // all the row-map loads in flight together, then clamped
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rr = r.row0 + min(wave * 8 * r.la + i * 8 + (lane >> 3), r.mrows - 1);
      r.arow[i] = row_token != nullptr && i < r.la ? row_token[rr] : rr;
    }
    if (row_token != nullptr) {
#pragma unroll
      for (int i = 0; i < 8; ++i) r.arow[i] = min(max(r.arow[i], 0), a_rows - 1);
    }
  };
  auto tile_src = [&](const TileRows& r, TileSrc& t) {
    int lane = threadIdx.x & 63;
    asm volatile("" : "+v"(lane));
    t.n_t = r.n_t;
    t.row0 = r.row0;
    t.mrows = r.mrows;
    // A: this lane's 16-byte chunk of row arow[i], at its swizzled place
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rl = wave * 8 * r.la + i * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(rl);
      t.a_src[i] = (const char*)(A + (size_t)r.arow[i] * K) + c * 16;
    }
    // B fragment j of k slice s: this lane's 16 bytes of block (nb_j, s). SwiGLU: j = 0 the
    // gate block, j = 1 the up block of the same 32 output columns (a pair tile: j = 2, 3
    // the same for n-tile n_t + 1).
#pragma unroll
    for (int j = 0; j < 2 * kNB; ++j) {
      const bf16_t* P;
      int nb;
      if (kTwoMat) { P = (j & 1) == 0 ? P0 : P1; nb = (r.n_t + (j >> 1)) * 4 + wn; }
      else { P = P0; nb = r.n_t * 8 + wn * 2 + (j & 1); }
      if (j >= kNB && !(kPairs && r.cls >= kPairTile)) nb = 0;   // not loaded
      t.bsrc[j] = P + ((size_t)r.e * NB + nb) * KS * 512 + lane * 8;
    }
  };
  // DMA instruction i of k-step kt for a class of LA loads per k-step and wave: rows
  // wave * 8 LA + 8 i + lane / 8, each at row * 128 bytes of the stage
  auto dma_for = [&](const TileSrc& t, auto la) {
    constexpr int LA = decltype(la)::value;
    return [&t, wave](int kt, bf16_t* stg, int i) {
      dma16_asm(t.a_src[i] + (uint32_t)(kt * BK * 2), lds_offset(stg) + (wave * LA + i) * 1024);
    };
  };

  // The tile's output from its accumulators (a slice of the split-K tail: a float32 partial
  // tile instead). Each kind has its own call site, so each gets its own register allocation.
  // acc holds the first NA fragments (rows 0 .. 32 NA - 1; the tile has no rows past them)
  auto epilogue = [&](auto& acc, int n_t, int row0, int mrows, float* part, auto slice) {
    constexpr bool kSlice = decltype(slice)::value;
    constexpr int NA = sizeof(acc) / sizeof(acc[0]);
    // acc[i][j][4q+s]: row m = i*32 + l32, column (within the wave's block j) = 8q + 4*lhi + s.
    if constexpr (kSlice) {   // float32 partial tile [BM][256], valid rows only
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int m = i * 32 + l32;
        if (m >= mrows) continue;
        float* prow = part + (size_t)m * 256;
#pragma unroll
        for (int j = 0; j < kNB; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int col = wn * 64 + j * 32 + 8 * q + 4 * lhi;
            *(float4*)(prow + col) = make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1],
                                                 acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
          }
      }
      return;
    }
    if constexpr (!kTwoMat) {
      // The 256 x 256 output tile leaves through LDS (the two A stages, free after the
      // barrier above), 64 rows at a time: the fragments' 8-byte pieces scatter over 32 rows
      // per store instruction, which made the stores of the previous tile, waited for in the
      // next prologue, a tenth of GEMM 2's time at short K. Read back in row order, every
      // store instruction writes two whole 512-byte rows. 16-byte chunk c of LDS row r sits
      // at c ^ (r & 31). LDS-only barriers: the global stores are never waited for here.
      constexpr int kRowB = 512;
      // Tile coordinates and lane index pass through empty asm, so no address below is
      // computed (and held in registers) across the k-loop.
      int e_row0 = row0, e_nt = n_t, e_mrows = mrows, e_lane = lane, e_tid = tid;
      asm volatile("" : "+s"(e_row0), "+s"(e_nt), "+s"(e_mrows));
      asm volatile("" : "+v"(e_lane), "+v"(e_tid));
      bf16_t* const ctile = C + (size_t)e_row0 * N + e_nt * 256;
      // pass p: fragments 2 p and 2 p + 1, rows 64 p .. 64 p + 63
#pragma unroll
      for (int p = 0; p < NA / 2; ++p) {
        char* buf = (char*)((p & 1) ? sa1 : sa0);
        const int lh = e_lane >> 5;
#pragma unroll
        for (int ii = 0; ii < 2; ++ii) {
          const int i = 2 * p + ii;
          const int lr = ii * 32 + (e_lane & 31);   // row of this lane's outputs in the block
#pragma unroll
          for (int j = 0; j < kNB; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float hv[4];
#pragma unroll
              for (int s = 0; s < 4; ++s)
                hv[s] = EPI == EPI_GELU ? gelu_f(acc[i][j][4 * q + s]) : acc[i][j][4 * q + s];
              // columns 8 chunk .. 8 chunk + 7 of the tile
              const int chunk = wn * 8 + j * 4 + q;
              *(uint2*)(buf + lr * kRowB + ((chunk ^ (lr & 31)) << 4) + lh * 8) = pack4(hv);
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int g = r * 256 + e_tid;     // 16-byte chunk of the 64 x 512-byte block
          const int row = g >> 5, chunk = g & 31;
          const int m = 64 * p + row;
          const uint4 v = *(const uint4*)(buf + row * kRowB + ((chunk ^ (row & 31)) << 4));
          if (m < e_mrows) *(uint4*)(ctile + (size_t)m * N + chunk * 8) = v;
        }
      }
      // every wave is done reading the stages before the next tile's DMA refills them
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      return;
    }
    // SwiGLU: h = silu(gate) * up, the gate and up columns of one output side by side in
    // the accumulators (j = 0 and j = 1)
    int e_lane = lane;
    asm volatile("" : "+v"(e_lane));
    const int l32 = e_lane & 31, lhi = e_lane >> 5;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int m = i * 32 + l32;
      if (m >= mrows) continue;
      bf16_t* crow = C + (size_t)(row0 + m) * N;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = n_t * 128 + wn * 32 + 8 * q + 4 * lhi;
        float hv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) hv[s] = silu_f(acc[i][0][4 * q + s]) * acc[i][1][4 * q + s];
        *(uint2*)(crow + col) = pack4(hv);
      }
    }
  };

  // One tile at a time: its loads, k-loop and epilogue (the single-matrix epilogues stage
  // their output through the two A stages, so the next tile's DMA waits for them).
  // The tile of an expert with at most 128 rows runs the same weight loads, waits and
  // barriers with only the first 4 A fragments (at most 64 rows: the first 2) and as many A
  // DMA loads per wave: a half (a quarter) of the MFMAs, fragment reads and token-row
  // loads, no accumulator for rows that are all padding. Each row
  // class is its own instantiation of the k-loop, so none carries a branch inside it. The
  // quarter class pays where small-expert tiles run beside large-expert ones (GEMM 2 of the
  // 32-expert workload 3-4% faster). (An expert's last, partial m-tile beside full ones
  // stays on the full path: finishing early, it pulled its block out of step with the
  // blocks sharing its weight panel through L2, measured 2-4% slower on Mixtral.)
  auto run_rows = [&](const TileSrc& t, int kb, int ke, float* part, auto slice, auto na) {
    constexpr int NA = decltype(na)::value;
    f32x16 acc[NA][kNB];
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int j = 0; j < kNB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    packed_kloop<NA, NA, kNB, NA>(kb, ke, sa0, sa1, t.bsrc, acc, load_a,
                                  dma_for(t, std::integral_constant<int, NA>{}));
    epilogue(acc, t.n_t, t.row0, t.mrows, part, slice);
  };
  // A pair tile: NA (4, or 2 for an expert of at most 64 rows) A fragments by 4 weight
  // fragments per slice (the k-loop's 2 x 2 form; at 4, the MFMAs of a full tile), then
  // each n-tile's outputs through the SwiGLU epilogue.
  auto run_pair = [&](const TileSrc& t, int kb, int ke, auto na) {
    constexpr int NA = decltype(na)::value;
    f32x16 acc[NA][2 * kNB];
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int j = 0; j < 2 * kNB; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    packed_kloop<NA, NA, 2 * kNB, NA>(kb, ke, sa0, sa1, t.bsrc, acc, load_a,
                                      dma_for(t, std::integral_constant<int, NA>{}));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x16 half[NA][kNB];
#pragma unroll
      for (int i = 0; i < NA; ++i)
#pragma unroll
        for (int j = 0; j < kNB; ++j) half[i][j] = acc[i][h * kNB + j];
      epilogue(half, t.n_t + h, t.row0, t.mrows, nullptr, std::false_type{});
    }
  };
  auto run_tile = [&](int tile, int kb, int ke, float* part, auto slice) {
    TileRows r;
    tile_rows(tile, r);
    TileSrc t;
    tile_src(r, t);
    if constexpr (kPairs) {
      if (r.cls == kPairTile) {
        run_pair(t, kb, ke, std::integral_constant<int, kNA / 2>{});
        return;
      }
      if (r.cls == kPairQuarter) {
        run_pair(t, kb, ke, std::integral_constant<int, kNA / 4>{});
        return;
      }
    }
    if (r.cls == kFull) run_rows(t, kb, ke, part, slice, std::integral_constant<int, kNA>{});
    else if (r.cls == kHalfRows) run_rows(t, kb, ke, part, slice, std::integral_constant<int, kNA / 2>{});
    else run_rows(t, kb, ke, part, slice, std::integral_constant<int, kNA / 4>{});
  };

  for (int base = 0; base < plan.full; base += gridDim.x) {
    const int tile = base + xcd * nper + li;
    if (tile >= plan.full) break;
    run_tile(tile, 0, KT, nullptr, std::false_type{});
  }
  if constexpr (EPI == EPI_NONE) {
    if (my_unit < plan.tail * plan.S) {
      int kb, ke;
      slice_range(KT, plan.S, my_unit % plan.S, kb, ke);
      run_tile(plan.full + my_unit / plan.S, kb, ke, partial + (size_t)my_unit * (BM * 256),
               std::true_type{});
    }
  }
}

hipError_t launch_pack_weight_bf16(const bf16_t* w, bf16_t* packed, int E, int K, int N,
                                   hipStream_t s) {
  const size_t chunks = (size_t)E * (N / 32) * (K / 16) * 64;
  const unsigned blocks = (unsigned)std::min<size_t>((chunks + 255) / 256, 16384);
  hipLaunchKernelGGL(pack_weight_kernel, dim3(blocks), dim3(256), 0, s, w, packed, E, K, N);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16_packed(int epi, const bf16_t* a, const int32_t* row_token,
                                   int a_rows, const int32_t* offsets, const bf16_t* p0,
                                   const bf16_t* p1, bf16_t* c, float* partial, int E, int K,
                                   int N, int max_rows, hipStream_t s) {
  const int outn = epi == EPI_SWIGLU ? 128 : 256;
  const bool split = epi == EPI_NONE && partial != nullptr;
  const long max_tiles = (long)((max_rows + BM - 1) / BM + E) * (N / outn);
  int grid = device_cus();
  grid = (grid / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  const long need = ((max_tiles + kXcds - 1) / kXcds) * kXcds;
  if (!split && need < grid) grid = (int)need;
  if (!split) partial = nullptr;
  const dim3 g(grid), b(256);
  switch (epi) {
    case EPI_SWIGLU:
      hipLaunchKernelGGL((grouped_gemm_packed_kernel<EPI_SWIGLU>), g, b, 0, s, a, row_token,
                         a_rows, offsets, p0, p1, c, partial, E, K, N, max_rows);
      break;
    case EPI_GELU:
      hipLaunchKernelGGL((grouped_gemm_packed_kernel<EPI_GELU>), g, b, 0, s, a, row_token,
                         a_rows, offsets, p0, p1, c, partial, E, K, N, max_rows);
      break;
    case EPI_NONE:
      hipLaunchKernelGGL((grouped_gemm_packed_kernel<EPI_NONE>), g, b, 0, s, a, row_token,
                         a_rows, offsets, p0, p1, c, partial, E, K, N, max_rows);
      break;
    default:
      return hipErrorInvalidValue;
  }
  if (split) {
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(1024), dim3(256), 0, s, partial, offsets, c, E,
                       K, N, max_rows, grid);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// Weight gradients with the second operand packed: for each expert e,
//   C_e[M][N] = sum over the padded rows k of expert e of A[k][m] B[k][n],
// with B given packed over the whole padded row space (pack_weight_kernel's layout with
// K = the packed rows, E = 1): block (nb, ks) holds B[16 ks + 8 (l >> 5) + q][32 nb + (l & 31)]
// in chunk l. B reduces over rows exactly as a weight reduces over k, so its fragments load
// straight into registers as in grouped_gemm_packed_kernel. A ([rows][lda], reduced over
// rows) goes global -> LDS by DMA as two [64 k][128 m] halves per k-step (the layout the
// plain forward kernel uses for weights) and reaches the MFMAs through transposing LDS
// reads. poff[e] .. poff[e+1] is expert e's padded row range, a multiple of 128 rows (whole
// pairs of k-steps), possibly empty (then C_e = 0); pad rows are zero. Tiles are ordered
// (expert, m-tile, n-tile) and run round by round: an XCD's blocks share A panels in L2,
// the XCDs of one round read the same expert's rows, and every block meets every expert in
// turn, which balances experts of different row counts. The k-loop is the one
// grouped_gemm_packed_kernel runs (packed_kloop), with the transposing A reads.
// TOUT: C is stored transposed, C_e^T [N][M] (dW_gate / dW_up computed as dg^T x).
template <bool TOUT>
__global__ __launch_bounds__(256, 1) void grouped_wgrad_packed_kernel(
    const bf16_t* __restrict__ A, int lda, const bf16_t* __restrict__ PB, int ksb,
    const int32_t* __restrict__ poff, bf16_t* __restrict__ C, int E, int M, int N) {
  __shared__ __attribute__((aligned(1024))) bf16_t sa0[BM * BK];
  __shared__ __attribute__((aligned(1024))) bf16_t sa1[BM * BK];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int MT = M / 256, NT = N / 256;
  const int total = E * MT * NT;
  const int xcd = blockIdx.x % kXcds, li = blockIdx.x / kXcds;
  const int nper = gridDim.x / kXcds;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, lhi = lane >> 5;
  // A in the stage as two [64 k][128 m] halves; fragment i covers 32 of the wave's 128 m
  const int krow0 = 8 * lhi + ((lane & 15) >> 2);
  uint32_t a_rd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c32 = ((32 * i) >> 4) + ((lane >> 4) & 1);
    a_rd[i] = (uint32_t)(wm * kHalf * 2) +
              (uint32_t)(krow0 * 256 + ((c32 ^ bswz(krow0)) << 5) + 8 * (lane & 3));
  }
  auto load_a = [&](const bf16_t* stg, int kk, FragA<4>& f) {
    const char* st = (const char*)stg + kk * 16 * 256;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const char* p = st + a_rd[i];
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const lds_char*)p);
      const v4i16 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const lds_char*)(p + 4 * 256));
      const v8i16 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      f.a[i] = __builtin_bit_cast(bf16x8, v);
    }
  };
  // DMA of A: instruction i of wave w fills rows k = (4w + i) * 4 .. + 3 of each half; lane
  // l loads 16-byte unit l & 15 of row 4(4w + i) + l / 16, stored swizzled
  uint32_t d_col[4];
  int d_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = (wave * 4 + i) * 4 + (lane >> 4);
    const int u = lane & 15;
    d_row[i] = k;
    d_col[i] = (uint32_t)((((u >> 1) ^ bswz(k)) << 4) + ((u & 1) << 3));
  }

  for (int base = 0, tile = xcd * nper + li; tile < total;
       base += gridDim.x, tile = base + xcd * nper + li) {
    const int e = tile / (MT * NT);
    const int rem = tile - e * MT * NT;
    const int m_t = rem / NT, n_t = rem - m_t * NT;
    const int kbase = __builtin_amdgcn_readfirstlane(poff[e]);
    const int KT = __builtin_amdgcn_readfirstlane((poff[e + 1] - poff[e]) / BK);
    const bf16_t* Ab = A + m_t * 256;
    const char* a_src[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a_src[i] = (const char*)(Ab + (size_t)(kbase + d_row[i]) * lda + d_col[i]);
    const bf16_t* bsrc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      bsrc[j] = PB + ((size_t)(n_t * 8 + wn * 4 + j) * ksb + kbase / 16) * 512 + lane * 8;
    constexpr int kLA = 8;   // A DMA loads per k-step and wave (4 rows x 2 halves)
    // DMA instruction q of k-step kt: row group q / 2, half q & 1
    auto dma_a = [&](int kt, bf16_t* stg, int q) {
      const size_t kA = (size_t)kt * BK * lda * 2;
      const uint32_t dst = lds_offset(stg) + wave * 4 * 1024;
      dma16_asm(a_src[q >> 1] + kA + (q & 1) * 256, dst + (q & 1) * kHalf * 2 + (q >> 1) * 1024);
    };
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    // A fragments come from two transposing reads each: 8 LDS reads per slice
    if (KT > 0) packed_kloop<kLA, 8>(0, KT, sa0, sa1, bsrc, acc, load_a, dma_a);   // KT even
    // acc[i][j][4q+s]: row m = wm*128 + 32i + l32, column n = wn*128 + 32j + 8q + 4lhi + s
    bf16_t* Ce = C + (size_t)e * M * N;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m_t * 256 + wm * 128 + i * 32 + l32;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n_t * 256 + wn * 128 + j * 32 + 8 * q + 4 * lhi;
          float v[4];
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) v[s2] = acc[i][j][4 * q + s2];
          if constexpr (TOUT) {
            // C^T[n][m]: for each of the four columns, lanes with consecutive m write
            // consecutive bytes of one row
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
              Ce[(size_t)(n + s2) * M + m] = (bf16_t)f32_to_bf16(v[s2]);
          } else {
            *(uint2*)(Ce + (size_t)m * N + n) = pack4(v);
          }
        }
    }
  }
}

hipError_t launch_wgrad_bf16_packed(const bf16_t* a, int lda, const bf16_t* pb, int kpack,
                                    const int32_t* poff, bf16_t* c, int E, int M, int N,
                                    int trans_out, hipStream_t s) {
  int grid = device_cus();
  grid = (grid / kXcds) * kXcds;
  if (grid < kXcds) grid = kXcds;
  const long need = (((long)E * (M / 256) * (N / 256) + kXcds - 1) / kXcds) * kXcds;
  if (need < grid) grid = (int)need;
  if (trans_out)
    hipLaunchKernelGGL((grouped_wgrad_packed_kernel<true>), dim3(grid), dim3(256), 0, s, a, lda,
                       pb, kpack / 16, poff, c, E, M, N);
  else
    hipLaunchKernelGGL((grouped_wgrad_packed_kernel<false>), dim3(grid), dim3(256), 0, s, a, lda,
                       pb, kpack / 16, poff, c, E, M, N);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------------
// float32 path: plain 16x16 LDS-tiled grouped GEMM on the vector ALUs (for fp32 layers).
constexpr int FT = 16;

template <int EPI>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(
    const float* __restrict__ A, const int32_t* __restrict__ row_token, int a_rows,
    const int32_t* __restrict__ offsets, const float* __restrict__ W0,
    const float* __restrict__ W1, float* __restrict__ C, int E, int K, int N, int max_rows) {
  __shared__ float As[FT][FT + 1], B0[FT][FT + 1], B1[FT][FT + 1];
  __shared__ int s_start[kMaxExperts + 1];
  __shared__ int s_perm[kMaxExperts];
  __shared__ int s_off[kMaxExperts + 1];
  __shared__ int s_wsum[4];
  int n_wide = 0;
  const int total = build_tile_starts<FT, false>(offsets, E, 1, max_rows, s_start, s_perm, s_off,
                                                 s_wsum, n_wide);
  const int tile = blockIdx.x;
  if (tile >= total) return;
  const int slot = find_expert(s_start, E, tile);   // list order is expert order here
  const int e = s_perm[slot];
  const int row_beg = s_off[e], m_e = s_off[e + 1] - row_beg;
  const int m_t = tile - s_start[slot];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int row = m_t * FT + ty;            // within the expert
  const int col = blockIdx.y * FT + tx;
  const float* We0 = W0 + (size_t)e * K * N;
  const float* We1 = (EPI == EPI_SWIGLU) ? W1 + (size_t)e * K * N : nullptr;
  size_t arow = 0;
  if (row < m_e)
    arow = row_token != nullptr ? (size_t)min(max(row_token[row_beg + row], 0), a_rows - 1)
                                : (size_t)(row_beg + row);
  float acc0 = 0.f, acc1 = 0.f;
  for (int k0 = 0; k0 < K; k0 += FT) {
    const int ka = k0 + tx, kb = k0 + ty;
    As[ty][tx] = (row < m_e && ka < K) ? A[arow * K + ka] : 0.f;
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

hipError_t launch_gemm_f32(int epi, const float* a, const int32_t* row_token, int a_rows,
                           const int32_t* offsets, const float* w0, const float* w1, float* c,
                           int E, int K, int N, int max_rows, hipStream_t s) {
  const dim3 g((max_rows + FT - 1) / FT + E, (N + FT - 1) / FT), b(256);
  switch (epi) {
    case EPI_SWIGLU:
      hipLaunchKernelGGL((grouped_gemm_f32_kernel<EPI_SWIGLU>), g, b, 0, s, a, row_token, a_rows, offsets, w0, w1, c, E, K, N, max_rows);
      break;
    case EPI_GELU:
      hipLaunchKernelGGL((grouped_gemm_f32_kernel<EPI_GELU>), g, b, 0, s, a, row_token, a_rows, offsets, w0, w1, c, E, K, N, max_rows);
      break;
    default:
      hipLaunchKernelGGL((grouped_gemm_f32_kernel<EPI_NONE>), g, b, 0, s, a, row_token, a_rows, offsets, w0, w1, c, E, K, N, max_rows);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
