// The k-loop of the packed-operand GEMMs (grouped_gemm_packed_kernel: token rows x packed
// weights; grouped_wgrad_packed_kernel: activations x packed rows), one implementation for
// both.
//
// Per 16-wide k slice a wave multiplies its four A fragments (from an LDS stage, filled by
// global->LDS DMA one k-step ahead) by four B fragments that come straight from global memory
// into registers: each is one 1 KB block of the packed layout, a coalesced 16-byte load per
// lane, issued one k-step ahead into a ring of eight slices. The loads are inline asm, so
// the compiler tracks none of them and adds no waits of its own (mixing LDS DMA and
// register loads, it would wait for all of them once per k-step); the loop instead executes
// the op lists of kloop_model.h and waits with the counts that model derives and checks at
// compile time.
#pragma once

#include <type_traits>
#include <utility>

#include "common.h"
#include "kloop_model.h"

namespace moe {

typedef __attribute__((address_space(3))) char lds_char_t;

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_char_t*)p;
}
// 16 bytes per lane global -> LDS at lds + 16 l. m0 is written right before the load that
// reads it, with the one wait state an LDS DMA needs after an SALU write of m0.
__device__ __forceinline__ void dma16_asm(const void* src, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(src), "s"(lds) : "memory", "m0");
}
// 16 bytes per lane global -> registers, from p + OFF bytes (OFF in the instruction's
// immediate field, so the slices of one k-step share one address computation).
template <int OFF>
__device__ __forceinline__ bf16x8 load16_asm_at(const bf16_t* p) {
  bf16x8 v;
  asm volatile("global_load_dwordx4 %0, %1, off offset:%2" : "=v"(v) : "v"(p), "n"(OFF) : "memory");
  return v;
}
// Wait until at most N of this wave's loads are in flight. The slice's NB fragments pass
// through the wait, so no instruction that reads them can be scheduled above it.
template <int N, int NB>
__device__ __forceinline__ void wait_loads(bf16x8* b) {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  static_assert(NB == 2 || NB == 4, "two or four fragments per slice");
  if constexpr (NB == 4)
    asm volatile("s_waitcnt vmcnt(%4)" : "+v"(b[0]), "+v"(b[1]), "+v"(b[2]), "+v"(b[3]) : "n"(N));
  else
    asm volatile("s_waitcnt vmcnt(%2)" : "+v"(b[0]), "+v"(b[1]) : "n"(N));
}
// s_waitcnt immediates: lgkmcnt(0) alone; vmcnt(n) with lgkmcnt(0)
constexpr int kWaitLgkm0Only = 0xC07F;
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4); }

// A fragments of one 16-wide k slice: rows (or columns) 32 i + (lane & 31) of the wave's
// 32 NA.
template <int NA>
struct FragA {
  bf16x8 a[NA];
};

template <class F, int... I>
__device__ __forceinline__ void for_each_op(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}

// The k-loop of one tile:
//   prologue(kb, ...)  issues A(kb), B slices 0..2 of kb, A(kb + 1), B slice 3 (kPrologue)
//   run(kb, ke, ...)   waits for A(kb), publishes it (kStart), then runs k-steps [kb, ke)
//                      (ke - kb even and >= 2) and ends with a barrier, after which both
//                      stages are free and no load of this wave is in flight
// Template and call arguments:
//   kLA      A DMA instructions per k-step and wave
//   kAReads  LDS read instructions per load_a (for the scheduling groups)
//   kLB, kNA B and A fragments per slice: 4 and 4 for a wave's 128 x 128 of the 2 x 2
//            layout, 2 and 8 for its 256 x 64 of the 1 x 4 one (2 and 4 for a tile of at
//            most 128 rows)
//   bsrc[j]  this lane's 16 bytes of B fragment j, slice 0 of k-step 0: slice s of k-step kt
//            is at bsrc[j] + 2048 kt elements + 1024 s bytes (the packed layout)
//   load_a(stage, kk, FragA&)  the wave's A fragments of slice kk from an LDS stage
//   dma_a(kt, stage, i)        this wave's global->LDS load i (0 .. kLA-1) of k-step kt
// acc[i][j] += B fragment j x A fragment i over the k-steps, v_mfma_f32_32x32x16_bf16 (each
// lane's accumulators then hold four consecutive columns j of one row i).
template <int kLA, int kAReads, int kLB = 4, int kNA = 4>
struct PackedKLoop {
  static_assert(kLB * kNA <= 16, "at most 16 MFMAs per slice: 256 accumulator registers");
  static_assert(kloop::tile_mismatches<kLA, kLB>() == 0 && kloop::counts_fit<kLA, kLB>(),
                "k-loop wait counts disagree with the issue order");
  // ring of k slices of B fragments (at most five live): slice s of k-step kt (counted from
  // the tile's first) in slot (4 kt + s) mod kloop::kRingSlots
  bf16x8 bv[kloop::kRingSlots][kLB];
  FragA<kNA> fr[2];           // A fragments of slices of even / odd index

  // B slice kk (0..3) of the k-step whose slice 0 is at base[j]
  template <int KK>
  __device__ __forceinline__ void load_b(const bf16_t* const* base, int slot) {
#pragma unroll
    for (int j = 0; j < kLB; ++j) bv[slot][j] = load16_asm_at<KK * 1024>(base[j]);
  }

  template <class DmaA>
  __device__ __forceinline__ void prologue(int kb, bf16_t* sa0, bf16_t* sa1,
                                           const bf16_t* const* bsrc, DmaA&& dma_a) {
    using namespace kloop;
    const bf16_t* pbase[kLB];   // slice 0 of k-step kb
#pragma unroll
    for (int j = 0; j < kLB; ++j) pbase[j] = bsrc[j] + (size_t)kb * 2048;
    for_each_op(
        [&](auto I) {
          constexpr Op op = kPrologue[decltype(I)::value];
          if constexpr (op.kind == kDmaA) {
#pragma unroll
            for (int q = 0; q < kLA; ++q) dma_a(kb + op.arg, op.arg ? sa1 : sa0, q);
          } else if constexpr (op.kind == kLoadB) {
            load_b<op.arg>(pbase, op.arg);
          } else {
            static_assert(op.kind == kDmaA, "op not allowed in the prologue");
          }
        },
        std::make_integer_sequence<int, kPrologueOps>{});
  }

  // kStart, then the k-steps [kb, ke) and a barrier.
  template <class LoadA, class DmaA>
  __device__ __forceinline__ void run(int kb, int ke, bf16_t* sa0, bf16_t* sa1,
                                      const bf16_t* const* bsrc, f32x16 (&acc)[kNA][kLB],
                                      LoadA&& load_a, DmaA&& dma_a) {
    using namespace kloop;
    auto mfma16 = [&](const FragA<kNA>& f, int slot) {
#pragma unroll
      for (int i = 0; i < kNA; ++i)
#pragma unroll
        for (int j = 0; j < kLB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[slot][j], f.a[i], acc[i][j], 0, 0, 0);
    };
    // MFMA m of a slice (m = kLB i + j)
    auto mfma_at = [&](const FragA<kNA>& f, const bf16x8* b, int m) {
      acc[m / kLB][m % kLB] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[m % kLB], f.a[m / kLB], acc[m / kLB][m % kLB], 0, 0, 0);
    };
    // Issue order inside a k-step. A wave issues in order, one instruction at a time, and an
    // MFMA occupies the matrix pipe for 32 cycles, during which the wave can issue other work;
    // a run of memory instructions between two MFMAs leaves the pipe idle. So each slice's
    // A fragment reads are spread over its MFMAs (one read, then kM / kAReads MFMAs), and
    // the last slice carries the k-step's refill DMAs, one batch after each of its first
    // kM - kAReads MFMAs, then the next stage's A reads over the rest. Measured against
    // issuing each group of memory instructions together: GEMM 1 / GEMM 2 -4.9% / -4.6%
    // (Mixtral), -5.7% / -1.9% (128 experts), bit-identical, the same fill traffic. The
    // load order, all the issue-order model sees, is unchanged.
    constexpr int kM = kLB * kNA;
    static_assert(kM % kAReads == 0 && kM > kAReads, "A reads spread over the slice's MFMAs");
    static_assert(kStep[kStepOps - 5].kind == kWaitB && kStep[kStepOps - 5].arg == 3 &&
                      kStep[kStepOps - 4].kind == kDmaA2 && kStep[kStepOps - 3].kind == kReadANext &&
                      kStep[kStepOps - 2].kind == kLoadBNext && kStep[kStepOps - 2].arg == 3 &&
                      kStep[kStepOps - 1].kind == kMfma && kStep[kStepOps - 1].arg == 3,
                  "the k-step ends with the sequence that runs interleaved");
    for_each_op(
        [&](auto I) {
          constexpr Op op = kStart[decltype(I)::value];
          if constexpr (op.kind == kWaitA0) {
            __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(start_count<kLA, kLB>()));
          } else if constexpr (op.kind == kBarrier) {
            __syncthreads();
          } else if constexpr (op.kind == kReadA0) {
            load_a(sa0, 0, fr[0]);
          } else {
            static_assert(op.kind == kWaitA0, "op not allowed in the start");
          }
        },
        std::make_integer_sequence<int, kStartOps>{});

    // k-step kt on stage `cur` (its B in ring slots sb .. sb + 3), `nxt` in flight, with R
    // k-steps left counting itself (capped at 3): a next k-step (kt + 1 < ke) for R >= 2, a
    // refill of `cur` (kt + 2 < ke) for R >= 3. sb and R are compile-time at every call
    // site, so the steady-state loop carries no branches and indexes the ring with
    // constants, which keeps the fragments in VGPRs and the accumulators in AGPRs.
    auto kstep = [&](int kt, bf16_t* cur, bf16_t* nxt, auto sbc, auto rem) {
      constexpr int sb = decltype(sbc)::value, R = decltype(rem)::value;
      constexpr bool kNext = R >= 2, kRefill = R >= 3;
      const bf16_t* nbase[kLB];   // slice 0 of k-step kt + 1
#pragma unroll
      for (int j = 0; j < kLB; ++j) nbase[j] = bsrc[j] + (size_t)(kt + 1) * 2048;
      for_each_op(
          [&](auto I) {
            constexpr int i = decltype(I)::value;
            constexpr Op op = kStep[i];
            constexpr int count = wait_count<kLA, kLB>(i, kNext, kRefill);
            if constexpr (op.kind == kLgkm0) {
              __builtin_amdgcn_s_waitcnt(kWaitLgkm0Only);
            } else if constexpr (op.kind == kWaitB) {
              wait_loads<count, kLB>(bv[wait_slot(sb, op.arg)]);
            } else if constexpr (op.kind == kReadA) {
              load_a(cur, op.arg, fr[op.arg & 1]);
            } else if constexpr (op.kind == kLoadBNext && op.arg < 3) {
              if constexpr (kNext) load_b<op.arg>(nbase, next_slot(sb, op.arg));
            } else if constexpr (op.kind == kMfma && op.arg < 3) {
              mfma16(fr[op.arg & 1], wait_slot(sb, op.arg));
              for_each_op([&](auto) {   // one A read, then kM / kAReads MFMAs
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, kM / kAReads, 0);
              }, std::make_integer_sequence<int, kAReads>{});
              __builtin_amdgcn_sched_barrier(0);
            } else if constexpr (op.kind == kLoadBNext || op.kind == kMfma ||
                                 op.kind == kReadANext) {
              // kReadANext, kLoadBNext 3 and kMfma 3: run inside the kDmaA2 sequence
            } else if constexpr (op.kind == kWaitANext) {
              if constexpr (count >= 0) __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(count));
              else __builtin_amdgcn_s_waitcnt(0);
            } else if constexpr (op.kind == kBarrier) {
              __syncthreads();
              __builtin_amdgcn_sched_barrier(0);
            } else if constexpr (op.kind == kDmaA2) {
              // kDmaA2, kReadANext, kLoadBNext 3, kMfma 3 as one sequence: the refill DMAs
              // (if any) kPer after each of slice 3's first kD MFMAs, then the next stage's A
              // reads spread over its last kAReads MFMAs, then slice 3 + 4 of the next k-step.
              // DMAs and B loads are inline asm, which the compiler does not move MFMAs
              // across; the A reads are ordinary LDS loads placed by the scheduling groups.
              const bf16x8* b3 = bv[wait_slot(sb, 3)];
              constexpr int kD = kM - kAReads;
              constexpr int kPer = (kLA + kD - 1) / kD;
              constexpr int kDmas = kRefill ? kLA : 0;
#pragma unroll
              for (int m = 0; m < kD; ++m) {
                mfma_at(fr[1], b3, m);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = m * kPer; q < (m + 1) * kPer; ++q)
                  if (q < kDmas) dma_a(kt + 2, cur, q);
                __builtin_amdgcn_sched_barrier(0);
              }
              if constexpr (kNext) load_a(nxt, 0, fr[0]);
#pragma unroll
              for (int m = kD; m < kM; ++m) mfma_at(fr[1], b3, m);
              if constexpr (kNext) {
                for_each_op([&](auto) {   // one A read, then one MFMA
                  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                  __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                }, std::make_integer_sequence<int, kAReads>{});
              }
              __builtin_amdgcn_sched_barrier(0);
              if constexpr (kNext) load_b<3>(nbase, next_slot(sb, 3));
            } else {
              static_assert(op.kind == kLgkm0, "op not allowed in a k-step");
            }
          },
          std::make_integer_sequence<int, kStepOps>{});
    };
    // The schedule (kloop_model.h, replayed there against the ring and the k-steps' order):
    // steady pairs while kt + 2 < ke (ke - kt is even, so both steps of such a pair have a
    // refill), then the last pair. An entry's stage is sa0 at an even offset.
    auto run_pair = [&](auto last, int kt0) {
      constexpr const StepSlot* t = decltype(last)::value ? kLastPair : kSteadyPair;
      for_each_op(
          [&](auto I) {
            constexpr StepSlot e = t[decltype(I)::value];
            const bool odd = e.off & 1;
            kstep(kt0 + e.off, odd ? sa1 : sa0, odd ? sa0 : sa1,
                  std::integral_constant<int, e.sb>{}, std::integral_constant<int, e.r>{});
          },
          std::make_integer_sequence<int, kPairSteps>{});
    };
    int kt = kb;
    for (; kt + 2 < ke; kt += kPairSteps) run_pair(std::false_type{}, kt);
    run_pair(std::true_type{}, kt);
    __syncthreads();   // every wave is done with both stages before the next tile's DMA
  }
};

// prologue immediately followed by run: one tile with nothing in between.
template <int kLA, int kAReads, int kLB = 4, int kNA = 4, class LoadA, class DmaA>
__device__ __forceinline__ void packed_kloop(int kb, int ke, bf16_t* sa0, bf16_t* sa1,
                                             const bf16_t* const* bsrc, f32x16 (&acc)[kNA][kLB],
                                             LoadA&& load_a, DmaA&& dma_a) {
  PackedKLoop<kLA, kAReads, kLB, kNA> loop;
  loop.prologue(kb, sa0, sa1, bsrc, dma_a);
  loop.run(kb, ke, sa0, sa1, bsrc, acc, load_a, dma_a);
}

}  // namespace moe
