// mxfp8.h -- the MXFP8 forward: quantisation folded into the dispatch and
// into the SwiGLU epilogue of the up projection, and the two expert GEMMs on
// the scaled matrix cores (MoK flash, §02: MXFP8 quantisation is fused into
// the dispatch, grouped GEMM and SwiGLU datapath).
//
// Data flow: every token row of x is quantised once along d (token-major
// codes [T, d] and scales [T, d/32]); the up-projection tiles pull their
// rows from there through the layout's source index, so the gathered copy
// of the rows is never written.  The SwiGLU output H is quantised along I
// in the up-projection epilogue (codes [R, I], scales [R, I/32]), which the
// down projection reads; its bf16 output rows are merged by the common
// combine.  Weights arrive quantised along their contraction axis (d for
// W1/W3, I for W2).
#pragma once

#include "gemm_mx.h"
#include "tasks_fwd.h"

namespace moe {

typedef TileMX<128, 128> TileMX128;  // 66 KB of LDS: two workgroups per CU

// Token block tb (kTokBlock tokens) of x, quantised along d.
__device__ void quant_tokens(const Fwd& F, int tb) {
  const int nbk = F.d / 32;
  const int t0 = tb * kTokBlock;
  const int nt = min(kTokBlock, F.T - t0);
  const bf16_t* X = (const bf16_t*)F.x;
  for (int i = threadIdx.x; i < nt * nbk; i += kThreads) {
    const int t = t0 + i / nbk, b = i - (i / nbk) * nbk;
    mx_quant_bf16_block(X + (size_t)t * F.d + 32 * b, F.xq + (size_t)t * F.d + 32 * b,
                        F.xs + (size_t)t * nbk + b);
  }
}

// Up projection + SwiGLU of one (row tile, column tile) in MXFP8; H is
// quantised in the epilogue, 32 columns of one row per block.
// CO as in g1_tile_bf16.
template <class TL, bool CO>
__device__ void g1_tile_mx(const Fwd& F, int tile, int nt, bf16_t* smem) {
  static_assert(TL::kMX, "MXFP8 tile");
  const TileRows tr = fwd_tile(F, tile);
  const int e = tr.e, r0 = tr.r0, n = tr.n;
  if (n <= 0) return;
  const int d = F.d, I = F.I, ds = d / 32;
  const uint8_t* W1 = (const uint8_t*)F.w1 + (size_t)e * I * d;
  const uint8_t* W3 = (const uint8_t*)F.w3 + (size_t)e * I * d;
  const uint8_t* S1 = F.w1s + (size_t)e * I * ds;
  const uint8_t* S3 = F.w3s + (size_t)e * I * ds;
  const int c0 = nt * (TL::BN / 2);
  KRowsMX<TL::BM, TL::BN> la;
  KRows<TL::BN> lb;
  auto wrow = [&](int nr, bool scale) -> const uint8_t* {
    int which, col;
    swiglu_brow<TL>(nr, which, col);
    if (scale) return (which ? S3 : S1) + (size_t)(c0 + col) * ds;
    return (which ? W3 : W1) + (size_t)(c0 + col) * d;
  };
  // rows past the tile's n repeat its last row (their outputs are dropped);
  // the source tokens come from the tile's own slot (written by its gather
  // task in this launch, on lines no other task writes)
  const int* ts = F.tsrc + slots::tile_slot(tile, 0, F.BM, 1);
  la.init([&](int r) { return F.xq + (size_t)clamp_token(ts[min(r, n - 1)], F.T) * d; },
          [&](int r) { return F.xs + (size_t)clamp_token(ts[min(r, n - 1)], F.T) * ds; },
          [&](int nr) { return wrow(nr, true); }, F.mx_wide1 != 0);
  lb.init([&](int nr) { return (const bf16_t*)wrow(nr, false); });
  f32x16_t acc[TL::MI][TL::NJ];
  tile_mainloop<TL>(d / 128, smem, acc, la, lb);

  // H in fp32 through LDS (row pitch 68 floats: the 16-byte reads of 16
  // consecutive rows below fall in 16 different bank groups)
  constexpr int W = TL::BN / 2, LD = W + 4, NBK = W / 32;
  static_assert((size_t)TL::BM * LD * 4 <= TL::smem_bytes, "H staging fits the tile's LDS");
  float* hs = (float*)smem;
  tile_visit_pairs<TL>(acc, [&](int row, int col, float av, float bv) { hs[row * LD + col] = silu_f(av) * bv; });
  __syncthreads();
  bf16_t* Hb = (bf16_t*)F.h;
  // H's codes and scales are read by the down projection, possibly in this
  // launch: stored coherently (kStoreCoherent)
  const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(wave_uniform(F.hq + (size_t)r0 * I + c0));
  const __amdgpu_buffer_rsrc_t rsc = buffer_rsrc(wave_uniform(F.hs + slots::tile_slot(tile, 0, F.BM, I / 32) + c0 / 32));
  for (int t = threadIdx.x; t < TL::BM * NBK; t += kThreads) {
    const int row = t % TL::BM, blk = t / TL::BM;
    if (row >= n) continue;
    float v[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 f = *(const float4*)(hs + row * LD + blk * 32 + 4 * q);
      v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
    }
    uint32_t w[8];
    const uint32_t sc = mx_quant32(v, w);
    const size_t r = (size_t)(r0 + row);
    if constexpr (CO) {
      const int qo = row * I + 32 * blk;
      store_coherent(rq, qo, make_uint4(w[0], w[1], w[2], w[3]));
      store_coherent(rq, qo + 16, make_uint4(w[4], w[5], w[6], w[7]));
      store_coherent_u8(rsc, row * (I / 32) + blk, (uint8_t)sc);
    } else {
      uint4* dst = (uint4*)(F.hq + r * I + c0 + 32 * blk);
      dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
      dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
      F.hs[slots::tile_slot(tile, row, F.BM, I / 32) + c0 / 32 + blk] = (uint8_t)sc;
    }
    if (Hb) {
      uint4* hb = (uint4*)(Hb + r * I + c0 + 32 * blk);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        hb[q] = make_uint4(pack_bf16x2(v[8 * q], v[8 * q + 1]), pack_bf16x2(v[8 * q + 2], v[8 * q + 3]),
                           pack_bf16x2(v[8 * q + 4], v[8 * q + 5]), pack_bf16x2(v[8 * q + 6], v[8 * q + 7]));
    }
  }
  // the saved pre-activations, when asked for (bf16)
  bf16_t* A = (bf16_t*)F.a;
  bf16_t* B = (bf16_t*)F.b;
  typedef Staged<TL::BM, TL::BN / 2> St;
  static_assert(St::bytes <= TL::smem_bytes, "staging fits the tile's LDS");
  const St st{smem};
  if (A) {
    __syncthreads();
    tile_visit_pairs<TL>(acc, [&](int row, int col, float av, float) { st.put(row, col, av); });
    st.flush(n, [&](int row) { return A + (size_t)(r0 + row) * I + c0; });
  }
  if (B) {
    __syncthreads();
    tile_visit_pairs<TL>(acc, [&](int row, int col, float, float bv) { st.put(row, col, bv); });
    st.flush(n, [&](int row) { return B + (size_t)(r0 + row) * I + c0; });
  }
}

// Down projection of one (row tile, column tile) in MXFP8, bf16 output rows.
template <class TL, bool CO>
__device__ void g2_tile_mx(const Fwd& F, int tile, int nt, bf16_t* smem) {
  static_assert(TL::kMX, "MXFP8 tile");
  const TileRows tr = fwd_tile(F, tile);
  const int e = tr.e, r0 = tr.r0, n = tr.n;
  if (n <= 0) return;
  const int d = F.d, I = F.I, is = I / 32;
  const uint8_t* W2 = (const uint8_t*)F.w2 + (size_t)e * d * I;
  const uint8_t* S2 = F.w2s + (size_t)e * d * is;
  const int c0 = nt * TL::BN;
  KRowsMX<TL::BM, TL::BN> la;
  KRows<TL::BN> lb;
  la.init([&](int r) { return F.hq + (size_t)(r0 + min(r, n - 1)) * I; },
          [&](int r) { return F.hs + slots::tile_slot(tile, min(r, n - 1), F.BM, is); },
          [&](int nr) { return S2 + (size_t)(c0 + nr) * is; }, F.mx_wide2 != 0);
  lb.init([&](int nr) { return (const bf16_t*)(W2 + (size_t)(c0 + nr) * I); });
  f32x16_t acc[TL::MI][TL::NJ];
  tile_mainloop<TL>(I / 128, smem, acc, la, lb);
  bf16_t* YP = (bf16_t*)F.yp;
  const Staged<TL::BM, TL::BN> st{smem};
  tile_visit<TL>(acc, [&](int row, int col, float v) { st.put(row, col, v); });
  if constexpr (CO)
    st.flush_coherent(n, YP + (size_t)r0 * d + c0, d);
  else
    st.flush(n, [&](int row) { return YP + (size_t)(r0 + row) * d + c0; });
}

// Standalone quantisation of [rows, K] bf16 along K: codes[r] and scales[r]
// from src row perm[r] / k (GATHER, the dispatch) or row r.
template <bool GATHER>
__global__ void __launch_bounds__(256) k_mx_quant_rows(const bf16_t* __restrict__ src, const int* __restrict__ perm,
                                                       int k, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, int64_t rows, int64_t K) {
  const int64_t nbk = K / 32, total = rows * nbk;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / nbk, b = i - r * nbk;
    // (a perm entry outside [0, rows) leaves its row unwritten)
    if (GATHER && (unsigned)perm[r] >= (unsigned)rows) continue;
    const int64_t s = GATHER ? (int64_t)(perm[r] / k) : r;
    mx_quant_bf16_block(src + s * K + 32 * b, codes + r * K + 32 * b, scales + i);
  }
}

// Token-major quantising gather: block b of token t is quantised once and
// its codes and scale written to each of the token's k rows (rows outside
// [0, R) skipped).  The same codes as quantising every gathered row, since
// the 32-element blocks lie within a row.
__global__ void __launch_bounds__(256) k_mx_quant_push(const bf16_t* __restrict__ x, const int* __restrict__ inv,
                                                       int k, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales, int T, int R, int d) {
  const int nbk = d / 32;
  const int64_t total = (int64_t)T * nbk;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < total; i += (int64_t)gridDim.x * kThreads) {
    const int64_t t = i / nbk, b = i - t * nbk;
    // every row index loaded before the first store (vmcnt counts stores
    // too, so a load between them would wait for the stores before it)
    int rows[kMaxK];
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) rows[j] = j < k ? inv[t * k + j] : -1;
    uint32_t w[8];
    const uint8_t s = mx_quant_bf16_words(x + t * d + 32 * b, w);
    const uint4 lo = make_uint4(w[0], w[1], w[2], w[3]), hi = make_uint4(w[4], w[5], w[6], w[7]);
#pragma unroll
    for (int j = 0; j < kMaxK; ++j) {
      const int r = rows[j];
      if ((unsigned)r >= (unsigned)R) continue;
      uint4* dst = (uint4*)(codes + (int64_t)r * d + 32 * b);
      dst[0] = lo;
      dst[1] = hi;
      scales[(int64_t)r * nbk + b] = s;
    }
  }
}

static int mx_quant_grid(int64_t blocks) {
  const int64_t g = (blocks + kThreads - 1) / kThreads;
  return (int)(g < 8192 ? g : 8192);
}

static int mxfp8_gather_perm(const bf16_t* x, const int* perm, uint8_t* xq, uint8_t* xs, int R, int d, int k,
                             hipStream_t st) {
  const int64_t blocks = (int64_t)R * (d / 32);
  hipLaunchKernelGGL(k_mx_quant_rows<true>, dim3(mx_quant_grid(blocks)), dim3(kThreads), 0, st, x, perm, k, xq,
                     xs, (int64_t)R, (int64_t)d);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

static int mxfp8_gather_push(const bf16_t* x, const int* inv, uint8_t* xq, uint8_t* xs, int T, int R, int d, int k,
                             hipStream_t st) {
  const int64_t blocks = (int64_t)T * (d / 32);
  hipLaunchKernelGGL(k_mx_quant_push, dim3(mx_quant_grid(blocks)), dim3(kThreads), 0, st, x, inv, k, xq, xs, T, R, d);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

static int mxfp8_quantize_rows(const bf16_t* src, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                               hipStream_t st) {
  const int64_t blocks = rows * (K / 32);
  hipLaunchKernelGGL(k_mx_quant_rows<false>, dim3(mx_quant_grid(blocks)), dim3(kThreads), 0, st, src,
                     (const int*)nullptr, 1, codes, scales, rows, K);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
