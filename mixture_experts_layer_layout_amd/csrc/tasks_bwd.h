// tasks_bwd.h -- the backward of the expert path (routing frozen) as tasks,
// run either as one kernel per step or inside one persistent kernel whose
// workgroups take tickets in dependency order (like the forward).
//
// MoK flash (the page "Cursor's MoK achieves 2.37x performance boost on
// NVIDIA GB300 NVL72"), §01: training adds two exchanges in the opposite
// direction; §02: the backward pulls the reverse-combine and pushes the
// reverse-dispatch.  On one GPU both are row moves through the layout:
//   pull reverse-combine  the dH GEMM reads dY rows through the layout
//                         (G[r] = dY[src[r]], never staged)
//   expert dgrad/wgrad    dHu = G W2_e;  dgate_r = <dHu_r, H_r>;
//                         dH = g_r dHu;  SwiGLU backward
//                         dA = dH * B * s(A) (1 + A (1 - s(A))),
//                         dB = dH * silu(A);
//                         dW2_e = (g G)_e^T H_e;
//                         dXp = dA W1_e + dB W3_e;
//                         dW1_e = dA_e^T Xp_e, dW3_e = dB_e^T Xp_e
//                         (Xp[r] = X[src[r]] read through the layout)
//   push reverse-dispatch dX[t] = sum_j dXp[inv[t k + j]]  (a fixed-order
//                         gather-sum, so the result is deterministic)
// Tasks, in ticket order, and what each waits for:
//   setup      row tiles and expert order from the saved offsets
//   rowprep    src[r] = perm[r] / k, g[r] = gate[perm[r]], and the pulls
//              Xp[r] = X[src[r]], gG[r] = g[r] dY[src[r]] (the operands
//              of the weight gradients, as plain rows)
//   dh         (row tile, I tile): dHu, dgate partial, dA | dB   [setup]
//   dw2        (expert, band of d, 8 column tiles of I)          [setup]
//   dxp        (row tile, d tile), K = 2I over [dA | dB]         [dh of the row tile]
//   dw13       (expert, band of I, 8 column tiles of d): dW1 and dW3 together
//                                                                [dh of the expert]
//   dx         kCombTok tokens: dX and dgate                     [every dxp]
// Weight-gradient tiles are taken in order of decreasing expert load so the
// longest tiles start first.
#pragma once

#include "plan.h"
#include "tasks_fwd.h"

namespace moe {

typedef Tile<128, 128> TileDH;  // row tiles: dh, dxp
// Row tiles holding at most 64 rows (the tail of an expert, or a whole
// lightly loaded expert) run on a 64-row tile of the same width: the same
// weight columns are streamed, with half the matrix-core work on padding.
typedef Tile<64, 128> TileDH64;
typedef Tile<128, 128> TileDW;  // weight-gradient tiles: dw2, dw13
constexpr int kPrepTok = 8;     // tokens per row-preparation task
constexpr int kWgradPerTicket = 8;  // column tiles per weight-gradient task (one band)
// Stages in registers ahead in dh and dxp.  Measured at the DeepSeek-V3
// Zipf step: 2 is best (dxp 5.8 ms); 3 and 4 cost the registers of a second
// workgroup per CU (dxp 7.7 and 11.6 ms).
#ifndef MOE_DGRAD_AHEAD
#define MOE_DGRAD_AHEAD 2
#endif
constexpr int kDgradAhead = MOE_DGRAD_AHEAD;


struct Bwd {
  int T, d, E, k, I, R, BM, max_tiles;
  int nNdh, nNdx, nW2m, nW2n, nW13m, nW13n, nRP, nC;
  const bf16_t* dy;
  const bf16_t* x;
  const bf16_t* w1;
  const bf16_t* w3;
  const bf16_t* w2;
  const float* gate;     // [T, k]
  const int* offsets;    // [E+1] the forward's (caller's) offsets
  int* eoff;             // [E+1] the same after bwd_setup checked them (all
                         // zero when they do not describe R rows)
  const int* perm;       // [R]
  const int* inv;        // [R]
  const bf16_t* a;       // [R, I]
  const bf16_t* b;       // [R, I]
  const bf16_t* h;       // [R, I]
  bf16_t* dx;            // [T, d]
  bf16_t* dw1;           // [E, I, d]
  bf16_t* dw3;           // [E, I, d]
  bf16_t* dw2;           // [E, d, I]
  float* dgate;          // [T, k]
  int* tile_e;           // [max_tiles]
  int* tile_r0;
  int* tile_n;
  int* etile;            // [E+1] first row tile of each expert
  int* eorder;           // [E] experts by decreasing row count
  int* src;              // [R]
  float* grow;           // [R]
  bf16_t* dab;           // [R, 2I]  dA | dB
  bf16_t* dxp;           // [R, d]
  float* dgp;            // [nNdh, R] dgate partial sums
  bf16_t* xp;            // [R, d] X pulled into expert order
  bf16_t* gg;            // [R, d] g_r * dY pulled into expert order
  const bf16_t* zrow;    // >= 2I + d + 256 zeros: the K tail of weight-gradient tiles
  // MXFP8 data gradients (null / 0 in the bf16 backward): the weights
  // transposed and quantised along the contraction axis of each product,
  // the upstream gradient and [dA | dB] quantised along their rows
  const uint8_t* w1t;    // [E, d, I] codes of W1^T, blocks along I
  const uint8_t* w3t;    // [E, d, I]
  const uint8_t* w2t;    // [E, I, d] codes of W2^T, blocks along d
  const uint8_t* w1ts;   // [E, d, I/32] scale codes
  const uint8_t* w3ts;
  const uint8_t* w2ts;   // [E, I, d/32]
  uint8_t* dyq;          // [T, d] codes of dY
  uint8_t* dys;          // [T, d/32]
  uint8_t* dabq;         // [R, 2I] codes of [dA | dB]
  uint8_t* dabs;         // [R, 2I/32]
  int mx_wide_d, mx_wide_i;  // scale rows read 4 stages at a time (KRowsMX)
  // MXFP8 weight gradients: their operands quantised along the rows (the
  // contraction axis) and stored transposed in row-tile slots: column c of
  // an operand holds local row i of row tile t at byte c * kcap + t * BM +
  // i (code 0 past the tile's rows), its scales at c * kcap / 32 + t * BM /
  // 32 + i / 32.  An expert's K range is its row tiles' slots.
  int mx;                // MXFP8 backward (rowprep then pulls no Xp, gG rows)
  int kcap;              // max_tiles * BM
  uint8_t* xT;           // [d, kcap]  x rows (through src)
  uint8_t* xTs;
  uint8_t* gT;           // [d, kcap]  g_r dY rows (through src)
  uint8_t* gTs;
  uint8_t* hT;           // [I, kcap]  H rows
  uint8_t* hTs;
  uint8_t* dabT;         // [2I, kcap] [dA | dB] rows
  uint8_t* dabTs;
  Sync s;
};

// ---------------------------------------------------------------- setup
// Row tiles and expert order from the saved offsets.  Offsets that do not
// describe R rows (offsets[0] = 0, nondecreasing, offsets[E] = R) record
// MOE_ERR_INVALID_ROUTE and are replaced by zeros: no row tile, every
// expert empty, so no task addresses a row past R.
__device__ void bwd_setup(const Bwd& B, int* sh /* >= 2*kMaxE + 16 ints */) {
  int* scnt = sh;
  int* stile = sh + kMaxE;
  int* tmp = sh + 2 * kMaxE;
  __shared__ int s_bad;
  if (threadIdx.x == 0) s_bad = (B.offsets[0] != 0 || B.offsets[B.E] != B.R) ? 1 : 0;
  __syncthreads();
  for (int e = threadIdx.x; e < B.E; e += kThreads)
    if (B.offsets[e + 1] < B.offsets[e]) s_bad = 1;
  __syncthreads();
  const bool bad = s_bad != 0;
  if (bad && threadIdx.x == 0) set_status(B.s.status, MOE_ERR_INVALID_ROUTE);
  for (int e = threadIdx.x; e <= B.E; e += kThreads) B.eoff[e] = bad ? 0 : B.offsets[e];
  for (int e = threadIdx.x; e < B.E; e += kThreads) {
    const int c = bad ? 0 : B.offsets[e + 1] - B.offsets[e];
    scnt[e] = c;
    stile[e] = cdiv(c, B.BM);
  }
  __syncthreads();
  const int ntiles = block_exclusive_scan(stile, B.E, tmp);
  for (int e = threadIdx.x; e < B.E; e += kThreads) {
    const int c = scnt[e], off = bad ? 0 : B.offsets[e];
    B.etile[e] = stile[e];
    for (int mt = 0, id = stile[e]; mt * B.BM < c; ++mt, ++id) {
      B.tile_e[id] = e;
      B.tile_r0[id] = off + mt * B.BM;
      B.tile_n[id] = min(B.BM, c - mt * B.BM);
    }
    // rank by (count descending, expert ascending)
    int rank = 0;
    for (int f = 0; f < B.E; ++f) {
      const int cf = scnt[f];
      rank += (cf > c) || (cf == c && f < e);
    }
    B.eorder[rank] = e;
  }
  if (threadIdx.x == 0) {
    B.etile[B.E] = ntiles;
    *B.s.n_mtiles = ntiles;
  }
}

// Token-major row preparation for kPrepTok tokens: each token's x and dY
// rows are read once and written to its k expert rows, dY scaled by the
// slot's gate (Xp[r] = x[t], G[r] = g dY[t] for r = inv[t k + j]); the row's
// source token and gate are recorded (all the MXFP8 backward needs).
__device__ void bwd_rowprep(const Bwd& B, int task) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nvec = B.d / 8;
  const int k = B.k;
  for (int tt = wave; tt < kPrepTok; tt += 4) {
    const int t = task * kPrepTok + tt;
    if (t >= B.T) break;
    // lane j < k holds slot j's row and gate
    const int lane_row = lane < k ? B.inv[(size_t)t * k + lane] : -1;
    const float lane_g = lane < k ? B.gate[(size_t)t * k + lane] : 0.0f;
    if (lane < k && (unsigned)lane_row < (unsigned)B.R) {  // inv entries outside [0, R) are skipped
      B.src[lane_row] = t;
      B.grow[lane_row] = lane_g;
    }
    if (B.mx) continue;  // the MXFP8 weight gradients quantise from x and dY through src
    wave_push_row((const uint4*)(B.x + (size_t)t * B.d), (uint4*)B.xp, nvec, k, B.R, lane_row,
                  [](int, uint4 u) { return u; });
    wave_push_row((const uint4*)(B.dy + (size_t)t * B.d), (uint4*)B.gg, nvec, k, B.R, lane_row, [&](int j, uint4 u) {
      const float g = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lane_g), j));
      uint32_t* w = (uint32_t*)&u;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        w[q] = pack_bf16x2(bf16_to_f32((bf16_t)(w[q] & 0xffff)) * g, bf16_to_f32((bf16_t)(w[q] >> 16)) * g);
      return u;
    });
  }
}

// ---------------------------------------------------------------- dh
// The dh epilogue of one (row tile, I tile) from the accumulators of dHu:
// the dgate partial sum of the tile's columns, dH = g dHu and the SwiGLU
// backward into [dA | dB] (shared by the bf16 and MXFP8 tiles, whose
// accumulator layouts are the same).  CO: a reader of [dA | dB] (dxp, dw13)
// runs in the same launch, so it is stored coherently (signal_add_stored).
template <class TL, bool CO = false>
__device__ __forceinline__ void bwd_dh_epilogue(const Bwd& B, f32x16_t (&acc)[TL::MI][TL::NJ], int r0, int n,
                                                int nt, bf16_t* smem) {
  const int I = B.I;
  const int c0 = nt * TL::BN;
  // dA staged in LDS (dB kept in the accumulators), then dB; the dgate
  // partial sums go through a small LDS area past the staging block
  typedef Staged<TL::BM, TL::BN> St;
  static_assert(St::bytes + 2 * TL::BM * sizeof(float) <= TL::smem_bytes, "dh staging fits the tile's LDS");
  const St st{smem};
  float* sred = (float*)(smem + TL::BM * St::LD);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  // Accumulator entries r and r + 1 (r even) are rows R and R + 1 of the
  // lane's column, and lanes 2m, 2m + 1 hold columns c, c + 1 of the same
  // rows: the even lane loads the 4-byte word of both columns in row R,
  // the odd lane that of row R + 1, and one lane-pair swap gives each the
  // value of its column in the other row (half the load instructions of
  // one 2-byte load per element, each moving twice the bytes).
  const bool odd = lane & 1;
  auto pair_of = [&](const bf16_t* base, size_t o, float& vr, float& vr1) {
    const uint32_t w = *(const uint32_t*)(base + o);
    const float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xffff0000u);
    const float own = odd ? hi : lo, got = swap_lane_pair(odd ? lo : hi);
    vr = odd ? got : own;
    vr1 = odd ? own : got;
  };
#pragma unroll
  for (int i = 0; i < TL::MI; ++i) {
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int row = wm * TL::WM + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const size_t gr0 = (size_t)(r0 + min(row, n - 1)), gr1 = (size_t)(r0 + min(row + 1, n - 1));
      const float g0 = B.grow[gr0], g1 = B.grow[gr1];
      const size_t grl = odd ? gr1 : gr0;
      float part0 = 0.0f, part1 = 0.0f;
#pragma unroll
      for (int j = 0; j < TL::NJ; ++j) {
        const int col = wn * TL::WN + 32 * j + (lane & 31);
        const size_t o = grl * I + c0 + (col & ~1);
        float a0, a1, b0, b1, h0, h1;
        pair_of(B.a, o, a0, a1);
        pair_of(B.b, o, b0, b1);
        pair_of(B.h, o, h0, h1);
        const float du0 = acc[i][j][r], du1 = acc[i][j][r + 1];
        part0 = fmaf(du0, h0, part0);
        part1 = fmaf(du1, h1, part1);
        const float dh0 = g0 * du0, dh1 = g1 * du1;
        const float sg0 = sigmoid_f(a0), sg1 = sigmoid_f(a1);
        st.put(row, col, dh0 * b0 * sg0 * (1.0f + a0 * (1.0f - sg0)));
        st.put(row + 1, col, dh1 * b1 * sg1 * (1.0f + a1 * (1.0f - sg1)));
        acc[i][j][r] = dh0 * a0 * sg0;
        acc[i][j][r + 1] = dh1 * a1 * sg1;
      }
      // sums over the 32 lanes holding these rows' columns (fixed tree)
#pragma unroll
      for (int o = 1; o < 32; o <<= 1) {
        part0 += __shfl_xor(part0, o);
        part1 += __shfl_xor(part1, o);
      }
      if ((lane & 31) == 0) {
        sred[wn * TL::BM + row] = part0;
        sred[wn * TL::BM + row + 1] = part1;
      }
    }
  }
  const size_t I2 = 2 * (size_t)I;
  if constexpr (CO)
    st.flush_coherent(n, B.dab + (size_t)r0 * I2 + c0, I2);
  else
    st.flush(n, [&](int row) { return B.dab + (size_t)(r0 + row) * I2 + c0; });
  if (threadIdx.x < TL::BM && (int)threadIdx.x < n) {
    const int row = threadIdx.x;
    B.dgp[(size_t)nt * B.R + r0 + row] = sred[row] + sred[TL::BM + row];
  }
  __syncthreads();
  tile_visit<TL>(acc, [&](int row, int col, float v) { st.put(row, col, v); });
  if constexpr (CO)
    st.flush_coherent(n, B.dab + (size_t)r0 * I2 + I + c0, I2);
  else
    st.flush(n, [&](int row) { return B.dab + (size_t)(r0 + row) * I2 + I + c0; });
}

// dHu = G W2_e for one (row tile, I tile), then the dh epilogue.
__device__ __forceinline__ TileRows bwd_tile(const Bwd& B, int tile) {
  return tile_rows(B.tile_e, B.tile_r0, B.tile_n, tile, B.max_tiles, B.E, B.R, B.BM);
}

template <class TL, bool CO>
__device__ void bwd_dh_tile_t(const Bwd& B, int tile, int nt, bf16_t* smem) {
  const TileRows tr = bwd_tile(B, tile);
  const int e = tr.e, r0 = tr.r0, n = tr.n;
  if (n <= 0) return;
  const int d = B.d, I = B.I;
  const bf16_t* W2 = B.w2 + (size_t)e * d * I;
  const int c0 = nt * TL::BN;
  KRows<TL::BM, kDgradAhead> la;
  // rows past n repeat the last row (their outputs are dropped)
  la.init([&](int r) -> const bf16_t* { return B.dy + (size_t)clamp_token(B.src[r0 + min(r, n - 1)], B.T) * d; });
  auto lb = kcols_n<TL::BN, kDgradAhead>([&](int kk, int) -> const bf16_t* { return W2 + (size_t)kk * I + c0; });
  f32x16_t acc[TL::MI][TL::NJ];
  tile_mainloop<TL, kDgradAhead>(d / 64, smem, acc, la, lb);
  bwd_dh_epilogue<TL, CO>(B, acc, r0, n, nt, smem);
}

template <bool CO = false>
__device__ void bwd_dh_tile(const Bwd& B, int tile, int nt, bf16_t* smem, float*) {
  if (bwd_tile(B, tile).n <= TileDH64::BM)
    bwd_dh_tile_t<TileDH64, CO>(B, tile, nt, smem);
  else
    bwd_dh_tile_t<TileDH, CO>(B, tile, nt, smem);
}

// ---------------------------------------------------------------- dxp
// dXp = [dA | dB] [W1_e ; W3_e] for one (row tile, d tile).
template <class TL>
__device__ void bwd_dxp_tile_t(const Bwd& B, int tile, int nt, bf16_t* smem) {
  const TileRows tr = bwd_tile(B, tile);
  const int e = tr.e, r0 = tr.r0, n = tr.n;
  if (n <= 0) return;
  const int d = B.d, I = B.I;
  const bf16_t* W1 = B.w1 + (size_t)e * I * d;
  const bf16_t* W3 = B.w3 + (size_t)e * I * d;
  const int c0 = nt * TL::BN;
  KRows<TL::BM, kDgradAhead> la;
  la.init([&](int r) -> const bf16_t* { return B.dab + (size_t)(r0 + min(r, n - 1)) * 2 * I; });
  auto lb = kcols_n<TL::BN, kDgradAhead>([&](int kk, int) -> const bf16_t* {
    return (kk < I ? W1 + (size_t)kk * d : W3 + (size_t)(kk - I) * d) + c0;
  });
  f32x16_t acc[TL::MI][TL::NJ];
  tile_mainloop<TL, kDgradAhead>(2 * I / 64, smem, acc, la, lb);
  const Staged<TL::BM, TL::BN> st{smem};
  tile_visit<TL>(acc, [&](int row, int col, float v) { st.put(row, col, v); });
  st.flush(n, [&](int row) { return B.dxp + (size_t)(r0 + row) * d + c0; });
}

__device__ void bwd_dxp_tile(const Bwd& B, int tile, int nt, bf16_t* smem) {
  if (bwd_tile(B, tile).n <= TileDH64::BM)
    bwd_dxp_tile_t<TileDH64>(B, tile, nt, smem);
  else
    bwd_dxp_tile_t<TileDH>(B, tile, nt, smem);
}

// A weight-gradient band: experts with at most 128 rows keep the band's A
// stages in LDS (tile_band), larger ones stream both operands.
template <class TL, class LA, class BP, class EPI>
__device__ __forceinline__ void wgrad_band(int nc, int nk, bf16_t* smem, LA& la, BP bptr, EPI& epi) {
  if (nk <= 2) {
    auto lb = kcols_n<TL::BN, 2>(bptr);
    lb.nk_ = nk;
    if (nk == 1)
      tile_band<TL, 1>(nc, smem, la, lb, epi);
    else
      tile_band<TL, 2>(nc, smem, la, lb, epi);
  } else {
    auto lb = kcols<TL::BN>(bptr);
    lb.nk_ = nk;
    tile_stream<TL>(nc, nk, smem, la, lb, epi);
  }
}

// ---------------------------------------------------------------- dw2
// dW2_e[n0 .. +128, i0 .. +128] = sum over the expert's rows r of
// gG[r, n] H[r, i] (gG pulled by rowprep): K = the expert's rows, k past
// them reads the zero row.  One task is
// a band of 128 output rows (n0) over kWgradPerTicket column tiles, streamed
// (tile_stream) so consecutive column tiles overlap.
__device__ void bwd_dw2_band(const Bwd& B, int rank, int task, bf16_t* smem) {
  typedef TileDW TL;
  const int e = min(max(B.eorder[min(rank, B.E - 1)], 0), B.E - 1);
  const int chunks = cdiv(B.nW2n, kWgradPerTicket);
  const int n0 = (task / chunks) * TL::BM;
  const int cb = (task % chunks) * kWgradPerTicket, nc = min(kWgradPerTicket, B.nW2n - cb);
  const int d = B.d, I = B.I;
  const int off = B.eoff[e], M = B.eoff[e + 1] - off;
  bf16_t* out = B.dw2 + (size_t)e * d * I + (size_t)n0 * I;
  auto epi = [&](int c, const f32x16_t (&acc)[TL::MI][TL::NJ]) {
    tile_store_staged<TL>(acc, [&](int wm) { return out + (size_t)(wm * TL::WM) * I + (cb + c) * TL::BN; }, I,
                          smem + TL::smem_bytes / sizeof(bf16_t));
  };
  if (M == 0) {
    f32x16_t zero[TL::MI][TL::NJ] = {};
    for (int c = 0; c < nc; ++c) epi(c, zero);
    return;
  }
  auto la = kcols<TL::BM>(
      [&](int kk, int) -> const bf16_t* { return kk < M ? B.gg + (size_t)(off + kk) * d + n0 : B.zrow; });
  auto bptr = [&](int kk, int c) -> const bf16_t* {
    return kk < M ? B.h + (size_t)(off + kk) * I + (cb + c) * TL::BN : B.zrow;
  };
  const int nk = cdiv(M, 64);
  la.nk_ = nk;
  wgrad_band<TL>(nc, nk, smem, la, bptr, epi);
}

// ---------------------------------------------------------------- dw13
// Rows 0..63 of a tile are dW1_e[i0 ..], rows 64..127 dW3_e[i0 ..]: both
// share the pulled X operand (Xp).  One task is a band (i0) over
// kWgradPerTicket column tiles of d, streamed like dw2.
__device__ void bwd_dw13_band(const Bwd& B, int rank, int task, bf16_t* smem) {
  typedef TileDW TL;
  const int e = min(max(B.eorder[min(rank, B.E - 1)], 0), B.E - 1);
  const int chunks = cdiv(B.nW13n, kWgradPerTicket);
  const int i0 = (task / chunks) * (TL::BM / 2);
  const int cb = (task % chunks) * kWgradPerTicket, nc = min(kWgradPerTicket, B.nW13n - cb);
  const int d = B.d, I = B.I;
  const int off = B.eoff[e], M = B.eoff[e + 1] - off;
  bf16_t* o1 = B.dw1 + (size_t)e * I * d + (size_t)i0 * d;
  bf16_t* o3 = B.dw3 + (size_t)e * I * d + (size_t)i0 * d;
  // wave row block 0 holds the dW1 rows, block 1 the dW3 rows
  static_assert(TL::WM == TL::BM / 2, "one wave row block per gradient");
  auto epi = [&](int c, const f32x16_t (&acc)[TL::MI][TL::NJ]) {
    tile_store_staged<TL>(acc, [&](int wm) { return (wm ? o3 : o1) + (cb + c) * TL::BN; }, d,
                          smem + TL::smem_bytes / sizeof(bf16_t));
  };
  if (M == 0) {
    f32x16_t zero[TL::MI][TL::NJ] = {};
    for (int c = 0; c < nc; ++c) epi(c, zero);
    return;
  }
  auto la = kcols<TL::BM>(
      [&](int kk, int) -> const bf16_t* { return kk < M ? B.dab + (size_t)(off + kk) * 2 * I + i0 : B.zrow; },
      I - TL::BM / 2);
  auto bptr = [&](int kk, int c) -> const bf16_t* {
    return kk < M ? B.xp + (size_t)(off + kk) * d + (cb + c) * TL::BN : B.zrow;
  };
  const int nk = cdiv(M, 64);
  la.nk_ = nk;
  wgrad_band<TL>(nc, nk, smem, la, bptr, epi);
}

// ---------------------------------------------------------------- dx
// dX[t] = sum_j dXp[inv[t k + j]] (fp32, slot order); dgate from the
// partial sums in column-tile order.  K as in combine_tokens_k.
template <int K>
__device__ void bwd_dx_tokens_k(const Bwd& B, int cb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int NR = K ? K : kMaxK;
  const int k = K ? K : B.k;
  const int nvec = B.d / 8;
  for (int tt = wave; tt < kCombTok; tt += 4) {
    const int t = cb * kCombTok + tt;
    if (t >= B.T) break;
    int rows[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) rows[j] = j < k ? clamp_row(B.inv[(size_t)t * k + j], B.R) : 0;
    {
      // dgate[t, j]: slot j's column-tile partials summed by a group of G
      // lanes (G the largest power of two with G k <= 64), each lane a
      // strided part, then a butterfly inside the group: a fixed order, and
      // the partial loads are issued by all lanes at once
      int G = 64;
      while (G * k > 64) G >>= 1;
      const int j = lane / G, q = lane - (lane / G) * G;
      float s = 0.0f;
      if (j < k) {
        const int r = clamp_row(B.inv[(size_t)t * k + j], B.R);
        for (int p = q; p < B.nNdh; p += G) s += B.dgp[(size_t)p * B.R + r];
      }
      for (int o = G >> 1; o > 0; o >>= 1) s += __shfl_xor(s, o);
      if (j < k && q == 0) B.dgate[(size_t)t * k + j] = s;
    }
    auto put = [&](int v, const float (&acc)[8]) {
      ((uint4*)B.dx)[(size_t)t * nvec + v] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                                        pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    };
    // known k: kCombVec vectors per lane per step, the next step's row
    // loads issued before this step's stores (as in combine_tokens_k)
    constexpr int VU = K ? kCombVec : 1;
    if constexpr (K != 0) {
      uint4 u[VU][K], nx[VU][K];
      auto load = [&](uint4 (&b)[VU][K], int v) {
#pragma unroll
        for (int h = 0; h < VU; ++h)
#pragma unroll
          for (int j = 0; j < K; ++j)
            if (v + 64 * h < nvec) b[h][j] = ((const uint4*)B.dxp)[(size_t)rows[j] * nvec + v + 64 * h];
      };
      load(u, lane);
      for (int v0 = lane; v0 < nvec; v0 += 64 * VU) {
        if (v0 + 64 * VU < nvec) load(nx, v0 + 64 * VU);
#pragma unroll
        for (int h = 0; h < VU; ++h) {
          if (v0 + 64 * h >= nvec) break;
          float acc[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
#pragma unroll
          for (int j = 0; j < K; ++j) {
            const bf16_t* p = (const bf16_t*)&u[h][j];
#pragma unroll
            for (int q = 0; q < 8; ++q) acc[q] += bf16_to_f32(p[q]);
          }
          put(v0 + 64 * h, acc);
        }
#pragma unroll
        for (int h = 0; h < VU; ++h)
#pragma unroll
          for (int j = 0; j < K; ++j) u[h][j] = nx[h][j];
      }
    } else {
      for (int v0 = lane; v0 < nvec; v0 += 64) {
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = 0.0f;
        for (int j = 0; j < k; ++j) {
          const uint4 u = ((const uint4*)B.dxp)[(size_t)rows[j] * nvec + v0];
          const bf16_t* p = (const bf16_t*)&u;
#pragma unroll
          for (int q = 0; q < 8; ++q) acc[q] += bf16_to_f32(p[q]);
        }
        put(v0, acc);
      }
    }
  }
}

__device__ void bwd_dx_tokens(const Bwd& B, int cb) {
  switch (B.k) {
    case 1: bwd_dx_tokens_k<1>(B, cb); break;
    case 2: bwd_dx_tokens_k<2>(B, cb); break;
    case 4: bwd_dx_tokens_k<4>(B, cb); break;
    case 6: bwd_dx_tokens_k<6>(B, cb); break;
    case 8: bwd_dx_tokens_k<8>(B, cb); break;
    default: bwd_dx_tokens_k<0>(B, cb); break;
  }
}

}  // namespace moe
