// router_bwd.h -- the router's backward through the gates.
//
// MoK flash §01: the router re-decides every step which experts a token goes
// to.  The choice is piecewise constant, so in training the gradient reaches
// the router only through the gates of the chosen experts.  With the choice
// frozen, for the gate logits z = x Wr^T + bias (no bias when it steers the
// selection only; it then gets no gradient), and gates divided by the routed
// scale c with c dgate as their gradient:
//   softmax, renormalised : dz_j = g_j (dg_j - sum_i g_i dg_i)
//   sigmoid, renormalised : dz_j = (dg_j - sum_i g_i dg_i) / S * s_j (1 - s_j),
//                           s = sigmoid(z), S = sum of the chosen s
//   sigmoid, plain        : dz_j = dg_j s_j (1 - s_j)
// and zero on every other logit; then dWr = dz^T x, dbias = sum_t dz and
// dx += dz Wr.  (A plain softmax reads every logit, so its gradient is dense;
// it is rejected on the host.)
//
// The sparsity is used directly: dx[t] gets k weighted rows of Wr (a
// gather-sum, like the combine), and dWr[e] is a weighted sum of the x rows
// routed to expert e, walked in the layout's expert order.  Every sum runs in
// a fixed order, so results are deterministic.
#pragma once

#include "common.h"

namespace moe {

constexpr int kRbSplits = 8;  // row splits per expert in the dWr sum

struct RouterBwd {
  int T, d, E, k, R, score, renorm;
  int select_only;      // the bias steered the selection only: z excludes it, no dbias
  float scale;          // routed scaling factor of the gates
  const void* x;        // act [T, d]
  const void* wr;       // act [E, d]
  const float* bias;    // [E] or null
  const float* logits;  // [T, E], bias not included
  const int* topk;      // [T, k]
  const float* gate;    // [T, k]
  const float* dgate;   // [T, k]
  const int* offsets;   // [E + 1]
  const int* perm;      // [R]
  float* dz;            // [R] workspace: dz of assignment a = t k + j
  float* dlogits;       // [T, E] or null
  float* part;          // [kRbSplits, E, d] workspace: dWr partial sums
  float* pbias;         // [kRbSplits, E] workspace: dbias partial sums
  void* dwr;            // act [E, d]
  float* dbias;         // [E] or null
  void* dx;             // act [T, d], added to
};

// One wave per token.  Lane j < k holds slot j: its expert, gate, dgate and
// biased logit; the slot sums are wave reductions (lanes >= k add zero).
// K = k when known at compile time (all k row loads of a vector in flight),
// 0 for any k.
template <class Act, int K>
__device__ void router_bwd_token(const RouterBwd& P, int t) {
  const int lane = threadIdx.x & 63;
  const int k = K ? K : P.k;
  const bool mine = lane < k;
  int e = 0;
  float g = 0.0f, dg = 0.0f, z = 0.0f;
  if (mine) {
    e = min(max(P.topk[(size_t)t * k + lane], 0), P.E - 1);  // saved indices clamped to [0, E)
    // the unscaled gate and the gradient it receives
    g = P.gate[(size_t)t * k + lane] / P.scale;
    dg = P.dgate[(size_t)t * k + lane] * P.scale;
    z = P.logits[(size_t)t * P.E + e] + (P.bias && !P.select_only ? P.bias[e] : 0.0f);
  }
  const float gdg = wave_sum(g * dg);
  float dzj;
  if (P.score == MOE_SCORE_SOFTMAX) {
    dzj = g * (dg - gdg);
  } else {
    const float s = sigmoid_f(z);
    if (P.renorm) {
      const float S = wave_sum(mine ? s : 0.0f);
      dzj = (dg - gdg) / S * s * (1.0f - s);
    } else {
      dzj = dg * s * (1.0f - s);
    }
  }
  if (!mine) dzj = 0.0f;
  if (mine) P.dz[(size_t)t * k + lane] = dzj;
  if (P.dlogits) {
    for (int c = lane; c < P.E; c += 64) {
      float v = 0.0f;
      for (int j = 0; j < k; ++j)
        if (__builtin_amdgcn_readlane(e, j) == c)
          v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dzj), j));
      P.dlogits[(size_t)t * P.E + c] = v;
    }
  }
  // dx[t] += sum_j dz_j Wr[e_j], fp32 in slot order
  constexpr int EPV = 16 / sizeof(Act);
  constexpr int NR = K ? K : kMaxK;
  const int nvec = P.d / EPV;
  const uint4* W = (const uint4*)P.wr;
  uint4* DX = (uint4*)P.dx;
  int ex[NR];
  float w[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    ex[j] = j < k ? __builtin_amdgcn_readlane(e, j) : 0;
    w[j] = j < k ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dzj), j)) : 0.0f;
  }
  for (int v = lane; v < nvec; v += 64) {
    const uint4 o = DX[(size_t)t * nvec + v];
    uint4 u[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j)
      if (K || j < k) u[j] = W[(size_t)ex[j] * nvec + v];
    float acc[EPV];
    const Act* po = (const Act*)&o;
#pragma unroll
    for (int q = 0; q < EPV; ++q) acc[q] = Elem<Act>::to_f32(po[q]);
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      if (!K && j >= k) break;
      const Act* p = (const Act*)&u[j];
#pragma unroll
      for (int q = 0; q < EPV; ++q) acc[q] = fmaf(w[j], Elem<Act>::to_f32(p[q]), acc[q]);
    }
    uint4 r;
    Act* pr = (Act*)&r;
#pragma unroll
    for (int q = 0; q < EPV; ++q) pr[q] = Elem<Act>::from_f32(acc[q]);
    DX[(size_t)t * nvec + v] = r;
  }
}

template <class Act>
__global__ void __launch_bounds__(256) k_router_bwd_tokens(RouterBwd P) {
  for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < P.T; t += gridDim.x * 4) {
    switch (P.k) {
      case 1: router_bwd_token<Act, 1>(P, t); break;
      case 2: router_bwd_token<Act, 2>(P, t); break;
      case 4: router_bwd_token<Act, 4>(P, t); break;
      case 8: router_bwd_token<Act, 8>(P, t); break;
      default: router_bwd_token<Act, 0>(P, t); break;
    }
  }
}

// Partial dWr and dbias of (expert e = blockIdx.x, column chunk blockIdx.y of
// 64 * EPV elements, row split blockIdx.z): the expert's rows are cut into
// kRbSplits consecutive ranges; wave w of the workgroup takes rows w, w+4,
// ... of its range (four rows in flight a step), and the four waves' sums
// are added in wave order.
template <class Act>
__global__ void __launch_bounds__(256) k_router_bwd_dwr(RouterBwd P) {
  constexpr int EPV = 16 / sizeof(Act);
  __shared__ float red[4][64 * EPV];
  __shared__ float redb[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x, ch = blockIdx.y, s = blockIdx.z;
  // the saved offsets clamped to [0, R] (rows outside are never read)
  const int lo0 = min(max(P.offsets[e], 0), P.R), n = max(min(max(P.offsets[e + 1], 0), P.R) - lo0, 0);
  const int lo = lo0 + (int)((int64_t)n * s / kRbSplits), hi = lo0 + (int)((int64_t)n * (s + 1) / kRbSplits);
  const int nvec = P.d / EPV;
  const int v = ch * 64 + lane;
  const bool col = v < nvec;
  const uint4* X = (const uint4*)P.x;
  float acc[EPV];
#pragma unroll
  for (int q = 0; q < EPV; ++q) acc[q] = 0.0f;
  float bsum = 0.0f;
  for (int r0 = lo + wave; r0 < hi; r0 += 16) {
    int a[4];
    float wz[4];
    uint4 u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = r0 + 4 * i < hi ? P.perm[r0 + 4 * i] : -1;
      a[i] = (unsigned)a[i] < (unsigned)P.R ? a[i] : -1;  // a perm entry outside [0, R) adds nothing
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wz[i] = a[i] >= 0 ? P.dz[a[i]] : 0.0f;
      if (a[i] >= 0 && col) u[i] = X[(size_t)(a[i] / P.k) * nvec + v];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (a[i] < 0) break;
      bsum += wz[i];
      if (col) {
        const Act* p = (const Act*)&u[i];
#pragma unroll
        for (int q = 0; q < EPV; ++q) acc[q] = fmaf(wz[i], Elem<Act>::to_f32(p[q]), acc[q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < EPV; ++q) red[wave][lane * EPV + q] = acc[q];
  if (lane == 0) redb[wave] = bsum;
  __syncthreads();
  if (wave == 0) {
    float* dst = P.part + ((size_t)s * P.E + e) * P.d + (size_t)v * EPV;
#pragma unroll
    for (int q = 0; q < EPV; ++q) {
      const float sum = ((red[0][lane * EPV + q] + red[1][lane * EPV + q]) + red[2][lane * EPV + q]) +
                        red[3][lane * EPV + q];
      if (col) dst[q] = sum;
    }
    if (ch == 0 && lane == 0) P.pbias[(size_t)s * P.E + e] = ((redb[0] + redb[1]) + redb[2]) + redb[3];
  }
}

// dWr[e, c] = sum over the splits in order; dbias[e] likewise.
template <class Act>
__global__ void __launch_bounds__(256) k_router_bwd_final(RouterBwd P) {
  const size_t n = (size_t)P.E * P.d;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    float sum = 0.0f;
    for (int s = 0; s < kRbSplits; ++s) sum += P.part[(size_t)s * n + i];
    ((Act*)P.dwr)[i] = Elem<Act>::from_f32(sum);
    if (P.dbias && i % P.d == 0) {
      const int e = (int)(i / P.d);
      float b = 0.0f;
      for (int s = 0; s < kRbSplits; ++s) b += P.pbias[(size_t)s * P.E + e];
      P.dbias[e] = P.select_only ? 0.0f : b;
    }
  }
}

}  // namespace moe
