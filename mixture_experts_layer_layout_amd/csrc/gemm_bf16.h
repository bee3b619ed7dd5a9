// gemm_bf16.h -- one workgroup tile of a bf16 GEMM on CDNA4 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate), used by every expert GEMM of
// the forward and backward.
//
// C[BM x BN] = sum_k A[m, k] * B[n, k], K consumed 64 at a time through two
// LDS stages (register prefetch of stage k+1 while stage k feeds the MFMAs,
// one barrier per step).  LDS holds both operands k-contiguous: a row of 64
// bf16 is 8 chunks of 16 bytes and chunk c of row r is stored at chunk
// c ^ (r & 7), so the 16-byte MFMA operand reads of 8 consecutive rows hit
// 8 different bank groups, as do the 16-byte stores of the loaders.
//
// Operands come through loaders that fill one LDS stage:
//   KRows   the operand is stored as rows with k contiguous (row-major
//           [rows, K]); rows may be gathered through an index (pull)
//   KCols   the operand is stored with k as the row index and the tile's
//           rows contiguous ([K, rows]); each thread loads an 8x8 block and
//           transposes it in registers before the LDS store
// Four waves split the tile 2 x 2; each wave owns (BM/2) x (BN/2) in
// (BM/64) x (BN/64) MFMA blocks of 32 x 32.
#pragma once

#include "common.h"

namespace moe {

__device__ __forceinline__ int lds_idx(int row, int chunk) {
  return (row << 6) + (((chunk ^ row) & 7) << 3);
}

template <int BM_, int BN_>
struct Tile {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int MI = WM / 32, NJ = WN / 32;
  static constexpr int LDS_A = BM * 64, LDS_B = BN * 64;
  static constexpr size_t smem_bytes = 2 * (LDS_A + LDS_B) * sizeof(bf16_t);
};

// ---------------------------------------------------------------- loaders
// Rows with k contiguous.  Thread t handles chunk t%8 of rows t/8 + 32*i.
template <int ROWS>
struct KRows {
  static constexpr int PER = ROWS / 32;
  const bf16_t* row[PER];
  uint4 v[PER];
  // rowptr(r) -> pointer to element k=0 of tile row r, or nullptr for a
  // row outside the operand (it loads as zeros).
  template <class F>
  __device__ __forceinline__ void init(F rowptr) {
    const int r0 = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < PER; ++i) row[i] = rowptr(r0 + 32 * i);
  }
  __device__ __forceinline__ void load(int kt) {
    const int ch = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if (row[i])
        v[i] = *(const uint4*)(row[i] + kt * 64 + ch * 8);
      else
        v[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds) const {
    const int r0 = threadIdx.x >> 3, ch = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < PER; ++i) *(uint4*)(lds + lds_idx(r0 + 32 * i, ch)) = v[i];
  }
};

// k is the row index of the stored operand; the tile's rows (ROWS of them)
// are contiguous within each stored row.  Thread t covers k-chunk t%8 and
// tile rows 8*(t/8) .. +7 (threads past ROWS/8*8 idle).
//   kptr(k) -> pointer to the stored row holding absolute k at the tile's
//              first row, or nullptr when k lies outside the operand
//   kscale(k) -> factor applied to that stored row (1 for none)
//   half_off  -> extra element offset for the second half of the tile's
//                rows (two column ranges of one stored row, e.g. the dA and
//                dB halves of [dA | dB]); 0 when the rows are contiguous
template <int ROWS>
struct KCols {
  static constexpr int NB = ROWS / 8;
  uint4 v[8];
  template <class P, class S>
  __device__ __forceinline__ void load(int kt, P kptr, S kscale, int half_off = 0) {
    const int kb = threadIdx.x & 7, nb = threadIdx.x >> 3;
    if (nb >= NB) return;
    const int coff = nb * 8 + (nb >= NB / 2 ? half_off : 0);
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int k = kt * 64 + kb * 8 + kk;
      const bf16_t* p = kptr(k);
      uint4 x = make_uint4(0, 0, 0, 0);
      if (p) {
        x = *(const uint4*)(p + coff);
        const float s = kscale(k);
        if (s != 1.0f) {
          uint32_t* w = (uint32_t*)&x;
#pragma unroll
          for (int q = 0; q < 4; ++q)
            w[q] = pack_bf16x2(bf16_to_f32((bf16_t)(w[q] & 0xffff)) * s,
                               bf16_to_f32((bf16_t)(w[q] >> 16)) * s);
        }
      }
      v[kk] = x;
    }
  }
  __device__ __forceinline__ void store(bf16_t* lds) const {
    const int kb = threadIdx.x & 7, nb = threadIdx.x >> 3;
    if (nb >= NB) return;
    const uint32_t* w = (const uint32_t*)v;  // w[kk*4 + q] = elements 2q, 2q+1 of k-row kk
#pragma unroll
    for (int mm = 0; mm < 8; ++mm) {
      // element mm of each k-row: dword mm/2, half mm%2
      const int q = mm >> 1;
      const uint32_t sel = (mm & 1) ? 0x07060302u : 0x05040100u;
      uint4 o;
      o.x = __builtin_amdgcn_perm(w[1 * 4 + q], w[0 * 4 + q], sel);
      o.y = __builtin_amdgcn_perm(w[3 * 4 + q], w[2 * 4 + q], sel);
      o.z = __builtin_amdgcn_perm(w[5 * 4 + q], w[4 * 4 + q], sel);
      o.w = __builtin_amdgcn_perm(w[7 * 4 + q], w[6 * 4 + q], sel);
      *(uint4*)(lds + lds_idx(nb * 8 + mm, kb)) = o;
    }
  }
};

// ---------------------------------------------------------------- core
template <class TL>
__device__ __forceinline__ void tile_compute(const bf16_t* As, const bf16_t* Bs,
                                             f32x16_t (&acc)[TL::MI][TL::NJ]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const int ch = ks * 2 + (lane >> 5);
    bf16x8_t a[TL::MI], b[TL::NJ];
#pragma unroll
    for (int i = 0; i < TL::MI; ++i)
      a[i] = *(const bf16x8_t*)(As + lds_idx(wm * TL::WM + 32 * i + (lane & 31), ch));
#pragma unroll
    for (int j = 0; j < TL::NJ; ++j)
      b[j] = *(const bf16x8_t*)(Bs + lds_idx(wn * TL::WN + 32 * j + (lane & 31), ch));
#pragma unroll
    for (int i = 0; i < TL::MI; ++i)
#pragma unroll
      for (int j = 0; j < TL::NJ; ++j) acc[i][j] = mfma32x32x16(a[i], b[j], acc[i][j]);
  }
}

// Runs the K loop.  LoadA(kt) / LoadB(kt) fetch stage kt into registers;
// StoreA(lds) / StoreB(lds) write the fetched stage.  nk may be 0.
template <class TL, class LA, class LB, class SA, class SB>
__device__ __forceinline__ void tile_mainloop(int nk, bf16_t* smem, f32x16_t (&acc)[TL::MI][TL::NJ],
                                              LA loadA, LB loadB, SA storeA, SB storeB) {
#pragma unroll
  for (int i = 0; i < TL::MI; ++i)
#pragma unroll
    for (int j = 0; j < TL::NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (nk <= 0) return;
  bf16_t* As = smem;
  bf16_t* Bs = smem + 2 * TL::LDS_A;
  __syncthreads();
  loadA(0);
  loadB(0);
  storeA(As);
  storeB(Bs);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      loadA(kt + 1);
      loadB(kt + 1);
    }
    tile_compute<TL>(As + cur * TL::LDS_A, Bs + cur * TL::LDS_B, acc);
    if (more) {
      storeA(As + (cur ^ 1) * TL::LDS_A);
      storeB(Bs + (cur ^ 1) * TL::LDS_B);
    }
    __syncthreads();
  }
}

// Visits every accumulator: f(tile_row, tile_col, value).
template <class TL, class F>
__device__ __forceinline__ void tile_visit(const f32x16_t (&acc)[TL::MI][TL::NJ], F f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < TL::MI; ++i)
#pragma unroll
    for (int j = 0; j < TL::NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * TL::WM + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wn * TL::WN + 32 * j + (lane & 31);
        f(row, col, acc[i][j][r]);
      }
}

// Paired visit for the SwiGLU tile: the B rows of wave column wn are laid
// out as [W1 cols | W3 cols] of the same (BN/4) output features, so block j
// and block j + NJ/2 hold the two pre-activations of one output.
// f(tile_row, out_col, a, b) with out_col in [0, BN/2).
template <class TL, class F>
__device__ __forceinline__ void tile_visit_pairs(const f32x16_t (&acc)[TL::MI][TL::NJ], F f) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int H = TL::NJ / 2;
#pragma unroll
  for (int i = 0; i < TL::MI; ++i)
#pragma unroll
    for (int j = 0; j < H; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * TL::WM + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int col = wn * (TL::WN / 2) + 32 * j + (lane & 31);
        f(row, col, acc[i][j][r], acc[i][j + H][r]);
      }
}

// Map a B-tile row of the SwiGLU tile to (which, out_col): which 0 = W1,
// 1 = W3; out_col in [0, BN/2).
template <class TL>
__device__ __forceinline__ void swiglu_brow(int n, int& which, int& col) {
  const int wn = n / TL::WN, w = n % TL::WN;
  which = w / (TL::WN / 2);
  col = wn * (TL::WN / 2) + (w % (TL::WN / 2));
}

}  // namespace moe
