// gemm_dma.h -- a bf16 tile whose row-major operands go from global memory
// straight into LDS (global_load_lds_dwordx4, 16 bytes a lane), through a
// ring of LDS slots: while slot s feeds the MFMAs, the loads of the next
// stages are in flight in the others.  No register staging and no LDS store
// instructions: the data path costs no VGPRs, so the loads in flight are
// bounded by LDS instead of by registers.  A 128 x 256 tile runs a ring of
// three 48 KB slots of 64 k values (two in flight); a 256 x 256 tile (a
// 128 x 128 block per wave, its accumulators in the AGPR half of the
// register file) a ring of four 32 KB slots of 32 k values (three in
// flight), twice the MFMA work per operand byte.  Both run one workgroup
// per CU.
//
// The LDS layout of a stage is the one of the register-staged tile
// (stage_idx), so tile_compute reads it unchanged.  A DMA instruction
// writes 64 lanes x 16 bytes to consecutive LDS bytes: with 64 k values a
// row (128 bytes, 8 chunks), lane i of the instruction that fills tile rows
// 8m .. 8m+7 lands at row 8m + i/8, slot i%8, and so loads the row's
// logical chunk (i%8) ^ key(row); with 32 (64 bytes, 4 chunks) an
// instruction fills 16 rows, lane i row 16m + i/4, slot i%4.
//
// Waiting: the DMA loads count in vmcnt like any vector load, and their LDS
// writes are complete when the count drops past them.  At the top of each
// step a wave waits until at most R - 2 stages of its own loads are still
// in flight (R slots), then the workgroup barrier makes every wave's part
// of the current stage visible, and also frees the slot the step refills
// (its readers finished before reaching the barrier).  The wait and the
// barrier are one asm statement with a memory clobber: the compiler's own
// waits know nothing of the DMA's LDS writes, and no memory access may move
// across.
#pragma once

#include <utility>

#include "gemm_bf16.h"

namespace moe {

#define MOE_LDS_PTR(p) ((void __attribute__((address_space(3)))*)(p))

template <int BM_, int BN_, int KS_ = 64, int SLOTS_ = 3>
struct TileD {
  static constexpr bool kMX = false;
  static constexpr bool kDMA = true;
  static constexpr bool kKeyHi = false;  // stage_key<KS, false>
  static constexpr int BM = BM_, BN = BN_, KS = KS_;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int MI = WM / 32, NJ = WN / 32;
  static constexpr int LDS_A = BM * KS, LDS_B = BN * KS;  // one stage, bf16 units
  static constexpr int SLOT = LDS_A + LDS_B;
  static constexpr int kSlots = SLOTS_;
  static_assert(kSlots >= 2 && kSlots <= 8, "a ring of two to eight slots");
  // the ring, or the epilogue's staged output block if that is larger
  static constexpr size_t ring_bytes = (size_t)kSlots * SLOT * sizeof(bf16_t);
  static constexpr size_t stage_out_bytes = (size_t)BM * (BN + 8) * sizeof(bf16_t);
  static constexpr size_t smem_bytes = ring_bytes > stage_out_bytes ? ring_bytes : stage_out_bytes;
  static_assert(smem_bytes <= 156 * 1024, "ring fits the CU's LDS beside the kernels' static LDS");
};

// Rows of an operand with k contiguous, loaded by DMA, KS k values a stage.
// Wave w issues PER instructions per stage; instruction q fills tile rows
// RPI m .. RPI m + RPI - 1, m = 4q + w.
template <int ROWS, int KS = 64>
struct DmaRows {
  static constexpr int CPR = KS / 8;         // 16-byte chunks per row and stage
  static constexpr int RPI = 64 / CPR;       // rows per instruction
  static constexpr int PER = ROWS / (4 * RPI);
  static_assert(PER * 4 * RPI == ROWS, "whole instructions per wave");
  const char* src[PER];
  // rowptr(r): element k = 0 of tile row r (readable for every r)
  template <class F>
  __device__ __forceinline__ void init(F rowptr) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int row = RPI * (4 * q + w) + lane / CPR;
      const int chunk = (lane % CPR) ^ stage_key<KS, false>(row);  // TileD::kKeyHi
      src[q] = (const char*)rowptr(row) + chunk * 16;
    }
  }
  // stage kt (KS k, 2 KS bytes of every row) into the operand's part of a slot
  __device__ __forceinline__ void issue(int kt, bf16_t* lds) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < PER; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(src[q] + (size_t)kt * (2 * KS)),
                                       MOE_LDS_PTR((char*)lds + (4 * q + w) * 1024), 16, 0, 0);
  }
};

// One step of a ring of R slots: wait for stage kt (slot SLOT; the R - 2
// later stages may stay in flight), refill the slot freed by stage kt-1
// with stage kt+R-1 (clamped: past the end it repeats the last stage), run
// the MFMAs of stage kt.
template <int SLOT, class TL, int NL>
__device__ __forceinline__ void dma_step(int kt, int last, bf16_t* smem, DmaRows<TL::BM, TL::KS>& A,
                                         DmaRows<TL::BN, TL::KS>& B, f32x16_t (&acc)[TL::MI][TL::NJ]) {
  constexpr int R = TL::kSlots;
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((R - 2) * NL) : "memory");
  bf16_t* nx = smem + ((SLOT + R - 1) % R) * TL::SLOT;
  const int ld = min(kt + R - 1, last);
  A.issue(ld, nx);
  B.issue(ld, nx + TL::LDS_A);
  __builtin_amdgcn_sched_barrier(0);
  bf16_t* cur = smem + SLOT * TL::SLOT;
  tile_compute<TL>(cur, cur + TL::LDS_A, acc);
}

// R consecutive steps from kt (slots 0 .. R-1), and the tail: the steps
// kt + s < nk of slots s < R - 1.
template <class TL, int NL, int... S>
__device__ __forceinline__ void dma_steps(int kt, int last, bf16_t* smem, DmaRows<TL::BM, TL::KS>& A,
                                          DmaRows<TL::BN, TL::KS>& B, f32x16_t (&acc)[TL::MI][TL::NJ],
                                          std::integer_sequence<int, S...>) {
  (dma_step<S, TL, NL>(kt + S, last, smem, A, B, acc), ...);
}
template <class TL, int NL, int... S>
__device__ __forceinline__ void dma_tail(int kt, int nk, int last, bf16_t* smem, DmaRows<TL::BM, TL::KS>& A,
                                         DmaRows<TL::BN, TL::KS>& B, f32x16_t (&acc)[TL::MI][TL::NJ],
                                         std::integer_sequence<int, S...>) {
  ((kt + S < nk ? dma_step<S, TL, NL>(kt + S, last, smem, A, B, acc) : void()), ...);
}

// The K loop over nk stages of TL::KS (nk may be 0: the tile is then zero).
// On return every DMA load has landed and every wave is past its last LDS
// read, so the caller may reuse the LDS (e.g. for a staged epilogue).
template <class TL>
__device__ __forceinline__ void tile_mainloop_dma(int nk, bf16_t* smem, f32x16_t (&acc)[TL::MI][TL::NJ],
                                                  DmaRows<TL::BM, TL::KS>& A, DmaRows<TL::BN, TL::KS>& B) {
  constexpr int R = TL::kSlots;
  constexpr int NL = DmaRows<TL::BM, TL::KS>::PER + DmaRows<TL::BN, TL::KS>::PER;  // loads per stage per wave
#pragma unroll
  for (int i = 0; i < TL::MI; ++i)
#pragma unroll
    for (int j = 0; j < TL::NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (nk <= 0) return;
  const int last = nk - 1;
  // the ring may still be read by the previous user of this LDS
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  // stages 0 .. R-2 into slots 0 .. R-2 (clamped like the steps' refills)
#pragma unroll
  for (int s = 0; s < R - 1; ++s) {
    A.issue(min(s, last), smem + s * TL::SLOT);
    B.issue(min(s, last), smem + s * TL::SLOT + TL::LDS_A);
  }
  int kt = 0;
  for (; kt + R <= nk; kt += R) dma_steps<TL, NL>(kt, last, smem, A, B, acc, std::make_integer_sequence<int, R>());
  dma_tail<TL, NL>(kt, nk, last, smem, A, B, acc, std::make_integer_sequence<int, R - 1>());
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace moe
