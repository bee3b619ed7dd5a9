// gemm_f32.h -- one workgroup tile of an fp32 GEMM with vector FMAs, for
// the fp32 layer (small shapes, correctness first).  Both operands are rows
// with k contiguous.  C[32 x 64]; thread t owns rows {t/16, t/16 + 16} and
// columns {t%16, t%16 + 16, t%16 + 32, t%16 + 48}, so columns c and c + 32
// (the two pre-activations of the SwiGLU tile) sit in the same thread.
#pragma once

#include "common.h"

namespace moe {

struct TileF32 {
  static constexpr int BM = 32, BN = 64, BK = 16;
  static constexpr size_t smem_bytes = (BM + BN) * (BK + 1) * sizeof(float);
};

// arow(r) / brow(n): pointer to element k=0 of tile row r / n, or nullptr
// (zeros).  K % 16 == 0.
template <class FA, class FB>
__device__ __forceinline__ void tile_f32(int K, float* smem, float (&acc)[2][4], FA arow, FB brow) {
  float* As = smem;                          // [BM][BK+1]
  float* Bs = smem + TileF32::BM * (TileF32::BK + 1);  // [BN][BK+1]
  const int t = threadIdx.x, tm = t >> 4, tn = t & 15;
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;
  // loader: A 32x16 = 512 values (2 per thread), B 64x16 = 1024 (4 per thread)
  const float* ap[2];
  const float* bp[4];
  for (int q = 0; q < 2; ++q) ap[q] = arow((t + 256 * q) >> 4);
  for (int q = 0; q < 4; ++q) bp[q] = brow((t + 256 * q) >> 4);
  const int kc = t & 15;
  for (int k0 = 0; k0 < K; k0 += TileF32::BK) {
    __syncthreads();
    for (int q = 0; q < 2; ++q) {
      const int r = (t + 256 * q) >> 4;
      As[r * (TileF32::BK + 1) + kc] = ap[q] ? ap[q][k0 + kc] : 0.0f;
    }
    for (int q = 0; q < 4; ++q) {
      const int n = (t + 256 * q) >> 4;
      Bs[n * (TileF32::BK + 1) + kc] = bp[q] ? bp[q][k0 + kc] : 0.0f;
    }
    __syncthreads();
    for (int kk = 0; kk < TileF32::BK; ++kk) {
      float a0 = As[tm * (TileF32::BK + 1) + kk];
      float a1 = As[(tm + 16) * (TileF32::BK + 1) + kk];
      for (int j = 0; j < 4; ++j) {
        float b = Bs[(tn + 16 * j) * (TileF32::BK + 1) + kk];
        acc[0][j] = fmaf(a0, b, acc[0][j]);
        acc[1][j] = fmaf(a1, b, acc[1][j]);
      }
    }
  }
  __syncthreads();
}

// f(row, col, v) over the tile.
template <class F>
__device__ __forceinline__ void tile_f32_visit(const float (&acc)[2][4], F f) {
  const int t = threadIdx.x, tm = t >> 4, tn = t & 15;
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 4; ++j) f(tm + 16 * i, tn + 16 * j, acc[i][j]);
}

// f(row, out_col, a, b) pairing column c with c + 32, out_col in [0, 32).
template <class F>
__device__ __forceinline__ void tile_f32_visit_pairs(const float (&acc)[2][4], F f) {
  const int t = threadIdx.x, tm = t >> 4, tn = t & 15;
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) f(tm + 16 * i, tn + 16 * j, acc[i][j], acc[i][j + 2]);
}

}  // namespace moe
