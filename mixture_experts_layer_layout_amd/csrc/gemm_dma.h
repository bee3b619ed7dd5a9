// gemm_dma.h -- a bf16 tile whose row-major operands go from global memory
// straight into LDS (global_load_lds_dwordx4, 16 bytes a lane), through a
// ring of three LDS slots: while slot s feeds the MFMAs, the loads of the
// next two stages are in flight in the other two.  No register staging and
// no LDS store instructions: the data path costs no VGPRs, so the loads in
// flight are bounded by LDS (three 48 KB slots for a 128 x 256 tile, one
// workgroup per CU) instead of by registers.
//
// The LDS layout of a stage is the one of the register-staged tile
// (lds_idx), so tile_compute reads it unchanged.  A DMA instruction writes
// 64 lanes x 16 bytes to consecutive LDS bytes; lane i of the instruction
// that fills tile rows 8m .. 8m+7 lands at row 8m + i/8, slot i%8, and so
// loads the row's logical 16-byte chunk (i%8) ^ lds_key<false>(row).
//
// Waiting: the DMA loads count in vmcnt like any vector load, and their LDS
// writes are complete when the count drops past them.  At the top of each
// step a wave waits until at most one stage of its own loads is still in
// flight, then the workgroup barrier makes every wave's part of the current
// stage visible, and also frees the slot the step refills (its readers
// finished before reaching the barrier).  The wait and the barrier are one
// asm statement with a memory clobber: the compiler's own waits know
// nothing of the DMA's LDS writes, and no memory access may move across.
#pragma once

#include "gemm_bf16.h"

namespace moe {

#define MOE_LDS_PTR(p) ((void __attribute__((address_space(3)))*)(p))

template <int BM_, int BN_>
struct TileD {
  static constexpr bool kMX = false;
  static constexpr bool kDMA = true;
  static constexpr bool kKeyHi = false;  // lds_key<false>
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int MI = WM / 32, NJ = WN / 32;
  static constexpr int LDS_A = BM * 64, LDS_B = BN * 64;  // one stage, bf16 units
  static constexpr int SLOT = LDS_A + LDS_B;
  static constexpr int kSlots = 3;
  static constexpr size_t smem_bytes = (size_t)kSlots * SLOT * sizeof(bf16_t);
  static_assert(smem_bytes <= 160 * 1024, "ring fits the CU's LDS");
};

// Rows of an operand with k contiguous, loaded by DMA.  Wave w issues
// PER instructions per stage; instruction q fills tile rows 8m .. 8m+7,
// m = 4q + w.
template <int ROWS>
struct DmaRows {
  static constexpr int PER = ROWS / 32;
  const char* src[PER];
  // rowptr(r): element k = 0 of tile row r (readable for every r)
  template <class F>
  __device__ __forceinline__ void init(F rowptr) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
      const int row = 8 * (4 * q + w) + (lane >> 3);
      const int chunk = (lane & 7) ^ lds_key<false>(row);  // TileD::kKeyHi
      src[q] = (const char*)rowptr(row) + chunk * 16;
    }
  }
  // stage kt (64 k, 128 bytes of every row) into the operand's part of a slot
  __device__ __forceinline__ void issue(int kt, bf16_t* lds) const {
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int q = 0; q < PER; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(src[q] + (size_t)kt * 128),
                                       MOE_LDS_PTR((char*)lds + (4 * q + w) * 1024), 16, 0, 0);
  }
};

// One step of the ring: wait for stage kt (slot SLOT), refill the slot freed
// by stage kt-1 with stage kt+2 (clamped: past the end it repeats the last
// stage), run the MFMAs of stage kt.
template <int SLOT, class TL, int NL>
__device__ __forceinline__ void dma_step(int kt, int last, bf16_t* smem, DmaRows<TL::BM>& A, DmaRows<TL::BN>& B,
                                         f32x16_t (&acc)[TL::MI][TL::NJ]) {
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NL) : "memory");
  bf16_t* nx = smem + ((SLOT + 2) % 3) * TL::SLOT;
  const int ld = min(kt + 2, last);
  A.issue(ld, nx);
  B.issue(ld, nx + TL::LDS_A);
  __builtin_amdgcn_sched_barrier(0);
  bf16_t* cur = smem + SLOT * TL::SLOT;
  tile_compute<TL>(cur, cur + TL::LDS_A, acc);
}

// The K loop over nk stages (nk may be 0: the tile is then zero).  On
// return every DMA load has landed and every wave is past its last LDS
// read, so the caller may reuse the LDS (e.g. for a staged epilogue).
template <class TL>
__device__ __forceinline__ void tile_mainloop_dma(int nk, bf16_t* smem, f32x16_t (&acc)[TL::MI][TL::NJ],
                                                  DmaRows<TL::BM>& A, DmaRows<TL::BN>& B) {
  constexpr int NL = DmaRows<TL::BM>::PER + DmaRows<TL::BN>::PER;  // loads per stage per wave
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
  A.issue(0, smem);
  B.issue(0, smem + TL::LDS_A);
  A.issue(min(1, last), smem + TL::SLOT);
  B.issue(min(1, last), smem + TL::SLOT + TL::LDS_A);
  int kt = 0;
  for (; kt + 3 <= nk; kt += 3) {
    dma_step<0, TL, NL>(kt, last, smem, A, B, acc);
    dma_step<1, TL, NL>(kt + 1, last, smem, A, B, acc);
    dma_step<2, TL, NL>(kt + 2, last, smem, A, B, acc);
  }
  if (kt < nk) dma_step<0, TL, NL>(kt, last, smem, A, B, acc);
  if (kt + 1 < nk) dma_step<1, TL, NL>(kt + 1, last, smem, A, B, acc);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace moe
