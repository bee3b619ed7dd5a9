// tasks_fwd.h -- the forward layer as tasks.  Each task is one workgroup's
// unit of work; the same functions run as separate kernels (one task per
// workgroup, the stream orders the steps) or inside the persistent kernel
// (tasks taken from a device-side ticket queue in dependency order, each
// waiting on the device counters its inputs raise).
//
// Steps (MoK flash = the page "Cursor's MoK achieves 2.37x performance boost
// on NVIDIA GB300 NVL72", by article section):
//   router_partial  router GEMM, one k-slice of 64 tokens x E experts
//   router_topk     sum of slices, top-k, gates, per-block expert bitmasks
//                   (§01: the router re-decides each token's experts)
//   layout_scan     per-expert counts, offsets, per-(block, expert) bases and
//                   the list of row tiles (§01: count first, then place, one
//                   expert's rows contiguous)
//   gather          each row tile derives its own source tokens from the
//                   masks and pulls the rows into expert order, then raises
//                   its ready counter (§02: pull dispatch; the communication
//                   side tells the compute side through GPU-local counters)
//   g1              up projection + SwiGLU for one (row tile, column tile)
//   g2              down projection for one (row tile, column tile)
//   combine         weighted merge back into token order (§01, §03)
#pragma once

#include <type_traits>

#include "common.h"
#include "gemm_bf16.h"
#include "gemm_dma.h"
#include "gemm_f32.h"

namespace moe {

constexpr int kTokBlock = 64;  // tokens per routing block (one mask bit each)
constexpr int kCombTok = 8;    // tokens per combine task
constexpr int kCombVec = 2;    // 16-byte vectors per lane per step of a combine row (known k)
constexpr int kMaxE = 1024;
constexpr int kMaxK = 16;

typedef Tile<128, 128> TileB128;   // 64 KB of LDS: two workgroups per CU
typedef Tile<256, 128> TileB256;
typedef TileD<128, 256> TileD256;  // direct-to-LDS ring, 144 KB: one workgroup per CU
// Row tiles of at most 64 rows (an expert's tail, or a whole lightly loaded
// expert) run on a 64-row tile of the same width: the same weight columns
// stream through the ring, with half the matrix-core work on padding.
typedef TileD<64, 256> TileD256h;
// 256-row stages: a 256 x 256 tile on a ring of four 32-k slots (half the
// operand bytes per MFMA of the 128-row tile, for experts with many rows);
// row tiles of at most 128 or 64 rows take the tiles above.
typedef TileD<256, 256, 32, 4> TileD256w;

struct Sync {
  int* queue;    // start of the counter region
  int* qctr;     // phase queues [kMaxPhases][8]
  int* abort;
  int* r2_done;
  int* scan_done;
  int* g2_done;
  int* n_mtiles;
  int* r1_cnt;   // [nb]
  int* ready;    // [max_tiles]
  int* h_cnt;    // [max_tiles]
  int* aux0;     // backward: [max_tiles]
  int* aux1;     // backward: [E]
  int* aux2;     // backward: [E]
  int* aux3;     // backward: scalar
  int* q_done;   // MXFP8 forward: token blocks quantised
  int32_t* status;
  long long spin_limit;
  uint32_t flags;  // moe_desc.flags (the test-only MOE_FLAG_TEST_* bits)
};

// The operands of one weighted merge: T tokens of k slots, rows of d
// elements.
struct Merge {
  int T, d, k, R;
  const void* yp;     // [R, d] expert outputs in expert order
  const float* gate;  // [T, k]
  const int* inv;     // [R]
  void* y;            // [T, d]
};

struct Fwd {
  int T, d, E, k, I, R, nb, S, BM, nN1, nN2, nC, max_tiles;
  int score, renorm, direct;
  int n_prod;  // workgroups [0, n_prod) of a persistent grid run only the
               // producer phases (routing, layout, gather, combine), the
               // others only the expert GEMMs; 0: every workgroup runs every
               // phase
  // routing options: bias for selection only, group-limited selection
  // (n_group > 1), factor on the gates
  int select_only, n_group, topk_group;
  float scale;
  const void* x;
  const void* wr;
  const float* bias;
  const void* w1;
  const void* w3;
  const void* w2;
  void* y;
  float* lpart;      // [S, lstride]: slice s holds [T, E] at s * lstride
  size_t lstride;    // T E rounded up to 32 floats: each slice starts on a line
  float* logits;     // [T, E] or null
  int* topk;         // [T, k]
  float* gate;       // [T, k]
  unsigned long long* bmask;  // [nb, E]
  int* bbase;        // [nb, E]
  int* counts;       // [E]
  int* offsets;      // [E+1]
  int* tile_e;       // [max_tiles]
  int* tile_r0;
  int* tile_n;
  int* etile;        // [E+1] first row tile of each expert (+ the total)
  int* perm;         // [R]
  int* inv;          // [R]
  int* tsrc;         // [max_tiles, BM]: source token of row i of row tile
                     // `tile` at tile * BM + i (each tile's slot on lines
                     // of its own: it is read inside the launch)
  float* grow;       // [R] gate of each row, or null
  void* xp;          // [R, d]
  void* a;           // [R, I] or null
  void* b;           // [R, I] or null
  void* h;           // [R, I]
  void* yp;          // [R, d]
  // MXFP8 (null otherwise): weight scales, token-major x codes/scales,
  // row-major H codes/scales
  const uint8_t* w1s;  // [E, I, d/32]
  const uint8_t* w3s;  // [E, I, d/32]
  const uint8_t* w2s;  // [E, d, I/32]
  uint8_t* xq;         // [T, d]
  uint8_t* xs;         // [T, d/32]
  uint8_t* hq;         // [R, I]
  uint8_t* hs;         // [max_tiles, BM, I/32]: H scales by row-tile slot
  // scale rows of the up / down projection read 16 bytes every 4 stages
  // (K % 512 == 0 and 16-byte aligned scale arrays)
  int mx_wide1, mx_wide2;
  // Macrobatches through a ring of two workspace slots: the merge of the
  // previous macrobatch (its expert outputs in the other slot, complete
  // when this launch starts) runs as extra tasks of this launch's first
  // phase, beside this macrobatch's routing.  prev.T = 0: none.
  Merge prev;
  int prev_nC;             // its combine tasks
  const int* prev_abort;   // its call's abort word (set: nothing to merge)
  Sync s;
};

__device__ __forceinline__ WaitCtx wctx(const Sync& s) { return WaitCtx{s.abort, s.status, s.spin_limit}; }

// The rows of row tile `tile`, clamped to the arrays they address: the tile
// id to [0, max_tiles), the expert to [0, E), the first row to [0, R] and the
// row count to [0, min(BM, R - r0)].  With a layout written by layout_scan
// (or bwd_setup) these are the values stored; the clamps keep a damaged
// workspace from turning into out-of-bounds addresses.
struct TileRows {
  int e, r0, n;
};
__device__ __forceinline__ TileRows tile_rows(const int* te, const int* tr0, const int* tn, int tile, int max_tiles,
                                              int E, int R, int BM) {
  tile = min(max(tile, 0), max_tiles - 1);
  TileRows t;
  t.e = min(max(te[tile], 0), E - 1);
  t.r0 = min(max(tr0[tile], 0), R);
  t.n = min(max(tn[tile], 0), min(BM, R - t.r0));
  return t;
}
__device__ __forceinline__ TileRows fwd_tile(const Fwd& F, int tile) {
  return tile_rows(F.tile_e, F.tile_r0, F.tile_n, tile, F.max_tiles, F.E, F.R, F.BM);
}

// A source token index read from the workspace, clamped to [0, T).
__device__ __forceinline__ int clamp_token(int t, int T) { return (unsigned)t < (unsigned)T ? t : 0; }
// A row index read from the workspace, clamped to [0, R).
__device__ __forceinline__ int clamp_row(int r, int R) { return (unsigned)r < (unsigned)R ? r : 0; }

// ---------------------------------------------------------------- router
// logits slice s of token block b: lpart[s][t][e] = sum over k in slice s.
// PF: the loads of the next 64-deep step are issued before this step's
// MFMAs (80 more VGPRs; the kernels whose other tasks leave only 256 a lane
// take the plain loop).
template <bool PF>
__device__ void router_partial_bf16(const Fwd& F, int task) {
  const int b = task / F.S, s = task % F.S;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int dk = F.d / F.S, k0 = s * dk;
  const int nEB = cdiv(F.E, 32);
  const bf16_t* X = (const bf16_t*)F.x;
  const bf16_t* Wr = (const bf16_t*)F.wr;
  const int koff = (lane >> 5) * 8;
  // wave w: rows 32 (w & 1) .. +31 of the block against expert blocks
  // REB (w >> 1) + 2 REB q .. +REB-1 (q = 0, 1, ..): the X fragment of a
  // 64-deep step is loaded once for REB expert blocks, and each pass over
  // the slice keeps REB accumulators (one pass for E <= 256).  Every
  // (row, expert) still sums its k in the same order.
  constexpr int REB = 4;
  const int rb = wave & 1;
  const int row = b * kTokBlock + rb * 32 + (lane & 31);
  const bool rv = row < F.T;
  const bf16_t* xa = X + (size_t)(rv ? row : 0) * F.d + k0 + koff;
  for (int eb0 = (wave >> 1) * REB; eb0 < nEB; eb0 += 2 * REB) {
    const bf16_t* wb[REB];
    bool ev[REB];
    f32x16_t acc[REB];
#pragma unroll
    for (int q = 0; q < REB; ++q) {
      const int e = (eb0 + q) * 32 + (lane & 31);
      ev[q] = e < F.E;
      wb[q] = Wr + (size_t)(ev[q] ? e : 0) * F.d + k0 + koff;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][r] = 0.0f;
    }
    bf16x8_t av[2][4], bv[2][REB][4];
    auto load = [&](int buf, int kk) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint4 ta = rv ? *(const uint4*)(xa + kk + 16 * u) : make_uint4(0, 0, 0, 0);
        av[buf][u] = *(const bf16x8_t*)&ta;
#pragma unroll
        for (int q = 0; q < REB; ++q) {
          const uint4 tb = ev[q] ? *(const uint4*)(wb[q] + kk + 16 * u) : make_uint4(0, 0, 0, 0);
          bv[buf][q][u] = *(const bf16x8_t*)&tb;
        }
      }
    };
    auto mma = [&](int buf) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int q = 0; q < REB; ++q) acc[q] = mfma32x32x16(av[buf][u], bv[buf][q][u], acc[q]);
    };
    if constexpr (PF) {
      load(0, 0);
      int kk = 0;
      for (; kk + 128 <= dk; kk += 128) {
        load(1, kk + 64);
        mma(0);
        if (kk + 128 < dk) load(0, kk + 128);
        mma(1);
      }
      if (kk < dk) mma(0);
    } else {
      for (int kk = 0; kk < dk; kk += 64) {
        load(0, kk);
        mma(0);
      }
    }
#pragma unroll
    for (int q = 0; q < REB; ++q) {
      const int e = (eb0 + q) * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int orow = b * kTokBlock + rb * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        // stored through the L2 (agent scope): the top-k tasks of this
        // launch read the slice on any XCD once signal_add_stored counts it
        if (orow < F.T && ev[q])
          __hip_atomic_store(F.lpart + (size_t)s * F.lstride + (size_t)orow * F.E + e, acc[q][r], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

__device__ void router_partial_f32(const Fwd& F, int task) {
  const int b = task / F.S, s = task % F.S;
  const int dk = F.d / F.S, k0 = s * dk;
  const float* X = (const float*)F.x;
  const float* Wr = (const float*)F.wr;
  for (int p = threadIdx.x; p < kTokBlock * F.E; p += kThreads) {
    const int row = b * kTokBlock + p / F.E, e = p % F.E;
    if (row >= F.T) continue;
    float acc = 0.0f;
    for (int kk = 0; kk < dk; ++kk) acc = fmaf(X[(size_t)row * F.d + k0 + kk], Wr[(size_t)e * F.d + k0 + kk], acc);
    __hip_atomic_store(F.lpart + (size_t)s * F.lstride + (size_t)row * F.E + e, acc, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <class Act, bool PF = true>
__device__ __forceinline__ void router_partial(const Fwd& F, int task) {
  if constexpr (std::is_same<Act, float>::value)
    router_partial_f32(F, task);
  else
    router_partial_bf16<PF>(F, task);
}

// Top-k of one token, one wave.  key (LDS) holds the E values ranked: the
// gate logits themselves, or score-space keys sigmoid(z) (+ a selection-only
// bias); row (LDS) holds the gate logits z.  Lane l owns experts l + 64 q.
// Largest key first; equal keys go to the lower expert index.  With
// n_group > 1 only experts of the topk_group best groups compete: lane g
// scores group g by the sum of its two largest keys, and the groups are
// taken best first (ties to the lower group).  Lane j < k returns the j-th
// choice and its gate (times scale).
__device__ __forceinline__ void wave_topk_gates(const float* row, const float* key, int E, int k, int score,
                                                int renorm, int n_group, int topk_group, float scale,
                                                int& sel_e, float& sel_g) {
  const int lane = threadIdx.x & 63;
  unsigned long long kept = ~0ull;  // groups whose experts compete
  int gs = E;
  if (n_group > 1) {
    gs = E / n_group;
    float gsc = -INFINITY;
    if (lane < n_group) {
      float t1 = -INFINITY, t2 = -INFINITY;
      for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
        float v = key[e];
        v = v != v ? -INFINITY : v;
        if (v > t1) { t2 = t1; t1 = v; } else if (v > t2) { t2 = v; }
      }
      gsc = gs > 1 ? t1 + t2 : t1;
    }
    kept = 0ull;
    for (int j = 0; j < topk_group; ++j) {
      float bv = ((kept >> lane) & 1ull) || lane >= n_group ? -INFINITY : gsc;
      int bi = lane < n_group && !((kept >> lane) & 1ull) ? lane : 0x7fffffff;
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
      }
      if (bi < 64) kept |= 1ull << bi;
    }
  }
  // experts of groups not kept start out as taken
  uint32_t taken = 0;
  if (n_group > 1)
    for (int e = lane, q = 0; e < E; e += 64, ++q)
      if (!((kept >> (e / gs)) & 1ull)) taken |= 1u << q;
  float sv = -INFINITY;
  sel_e = -1;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int e = lane, q = 0; e < E; e += 64, ++q) {
      float v = key[e];
      v = v != v ? -INFINITY : v;  // a NaN key ranks last, so k experts are always found
      if (!((taken >> q) & 1u) && (v > bv || (v == bv && e < bi))) { bv = v; bi = e; }
    }
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) sel_e = bi;
  }
  const bool mine = lane < k;
  if (mine) sv = row[sel_e];  // the chosen gate logit
  float g;
  if (score == MOE_SCORE_SOFTMAX) {
    const float m = __shfl(sv, 0);  // the largest logit
    if (renorm) {
      const float ex = mine ? expf(sv - m) : 0.0f;
      g = ex / wave_sum(ex);
    } else {
      float part = 0.0f;
      for (int e = lane; e < E; e += 64) part += expf(row[e] - m);
      g = (mine ? expf(sv - m) : 0.0f) / wave_sum(part);
    }
  } else {
    const float sg = mine ? 1.0f / (1.0f + expf(-sv)) : 0.0f;
    g = renorm ? sg / wave_sum(sg) : sg;
  }
  sel_g = g * scale;
}

constexpr int kTopkChunk = 8;   // tokens of one top-k task (staged in LDS at once)
constexpr int kTopkChunks = 64 / kTopkChunk;  // top-k tasks per 64-token block
// LDS of router_topk: the chunk's choices (within the first kMaxE u64) + a
// chunk of logits + one row of score-space keys per wave
constexpr size_t kTopkSmem = kMaxE * 8 + (size_t)kTopkChunk * kMaxE * 4 + 4 * (size_t)kMaxE * 4;

// One task per chunk of kTopkChunk tokens (kTopkChunks tasks per 64-token
// block): sums the slices, adds the bias, selects, writes idx/gates and
// (MASKS) its byte of every expert's block bitmask -- bits 8c .. 8c+7 of
// bmask[b, e] for chunk c, zeros included, so no task needs the mask
// cleared first and no two tasks write the same byte.  The logits of the
// chunk's tokens are summed into LDS by the whole workgroup (coalesced,
// independent loads), then each wave selects for 2 of them.  With S == 1
// and lpart == the caller's logits this is also the standalone route step.
template <bool MASKS>
__device__ void router_topk(const Fwd& F, int task, char* smem) {
  int* ssel = (int*)smem;  // [kTopkChunk][kMaxK] chosen experts of the chunk
  float* sv = (float*)(smem + kMaxE * 8);
  float* skey = sv + kTopkChunk * kMaxE + (threadIdx.x >> 6) * kMaxE;  // this wave's keys
  const bool keyed = F.select_only || F.n_group > 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int E = F.E;
  const int b = task / kTopkChunks, c = task - b * kTopkChunks;
  const int t0 = b * kTokBlock + c * kTopkChunk;
  __syncthreads();
  if (t0 < F.T) {
    for (int p = threadIdx.x; p < kTopkChunk * E; p += kThreads) {
      const int t = t0 + p / E, e = p % E;
      if (t >= F.T) break;
      float v = 0.0f;
      for (int s = 0; s < F.S; ++s) v += F.lpart[(size_t)s * F.lstride + (size_t)t * E + e];
      if (F.logits) F.logits[(size_t)t * E + e] = v;
      if (F.bias && !F.select_only) v += F.bias[e];
      sv[p] = v;
    }
    __syncthreads();
    for (int tt = wave; tt < kTopkChunk; tt += 4) {
      const int t = t0 + tt;
      if (t >= F.T) break;
      int se;
      float sg;
      const float* row = sv + tt * E;
      if (keyed) {
        // score-space keys sigmoid(z) (+ the selection-only bias); the
        // wave's own LDS row, written and read by this wave only
        for (int e = lane; e < E; e += 64)
          skey[e] = 1.0f / (1.0f + expf(-row[e])) + (F.select_only && F.bias ? F.bias[e] : 0.0f);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      wave_topk_gates(row, keyed ? skey : row, E, F.k, F.score, F.renorm, F.n_group, F.topk_group, F.scale,
                      se, sg);
      if (lane < F.k) {
        // indices, gates and mask bytes are stored through the L2 (agent
        // scope), as the router's slices: the layout and gather tasks of
        // this launch read them on any XCD once signal_add_stored counts them
        __hip_atomic_store(F.topk + (size_t)t * F.k + lane, se, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(F.gate + (size_t)t * F.k + lane, sg, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (MASKS) ssel[tt * kMaxK + lane] = se;
      }
    }
  }
  if (MASKS) {
    __syncthreads();
    const int nt = max(0, min(kTopkChunk, F.T - t0));  // tokens of this chunk
    for (int e = threadIdx.x; e < E; e += kThreads) {
      unsigned int byte = 0;
      for (int tt = 0; tt < nt; ++tt)
        for (int j = 0; j < F.k; ++j)
          if (ssel[tt * kMaxK + j] == e) byte |= 1u << tt;
      __hip_atomic_store((uint8_t*)(F.bmask + (size_t)b * E + e) + c, (uint8_t)byte, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Expert bitmasks of one token block from given indices (the layout entry
// point).  Out-of-range or repeated experts set MOE_ERR_INVALID_ROUTE.
__device__ void build_masks(const Fwd& F, int b, unsigned long long* smask) {
  for (int e = threadIdx.x; e < F.E; e += kThreads) smask[e] = 0ull;
  __syncthreads();
  for (int p = threadIdx.x; p < kTokBlock * F.k; p += kThreads) {
    const int tt = p / F.k, t = b * kTokBlock + tt;
    if (t >= F.T) continue;
    const int e = F.topk[(size_t)t * F.k + p % F.k];
    if (e < 0 || e >= F.E) {
      set_status(F.s.status, MOE_ERR_INVALID_ROUTE);
      continue;
    }
    const unsigned long long bit = 1ull << tt;
    if (atomicOr(&smask[e], bit) & bit) set_status(F.s.status, MOE_ERR_INVALID_ROUTE);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < F.E; e += kThreads) {
    const unsigned long long m = smask[e];
    F.bmask[(size_t)b * F.E + e] = m;
  }
}

// ---------------------------------------------------------------- layout
// Exclusive scan of n <= 1024 ints in LDS (in place), returns the total.
__device__ int block_exclusive_scan(int* v, int n, int* tmp /* >= 8 ints */) {
  const int per = cdiv(n, kThreads);
  const int lo = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (lo + i < n) local += v[lo + i];
  // inclusive scan of `local` across the block
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = local;
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  int wbase = 0, total = 0;
  for (int w = 0; w < 4; ++w) {
    if (w < wave) wbase += tmp[w];
    total += tmp[w];
  }
  int run = wbase + x - local;
  for (int i = 0; i < per; ++i)
    if (lo + i < n) {
      const int c = v[lo + i];
      v[lo + i] = run;
      run += c;
    }
  __syncthreads();
  return total;
}

// An int of the layout: with COH (a persistent launch whose other tasks
// read the layout on any XCD once signal_add_stored counts it) stored
// through the L2 at agent scope, else an ordinary store (the standalone
// layout kernel: the launch boundary publishes it).
template <bool COH>
__device__ __forceinline__ void st_layout(int* p, int v) {
  if constexpr (COH)
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else
    *p = v;
}

// One workgroup: counts, offsets, bases, tile list.  The masks of a valid
// routing hold exactly R = T k bits and give at most max_tiles row tiles;
// anything else (a repeated or out-of-range expert given to moe_layout)
// records MOE_ERR_INVALID_ROUTE and publishes no row tile, so no later task
// addresses a row past R.
template <bool COH>
__device__ void layout_scan(const Fwd& F, int* sh /* >= 2*kMaxE + 16 ints */) {
  int* scnt = sh;
  int* stile = sh + kMaxE;
  int* tmp = sh + 2 * kMaxE;
  __syncthreads();
  for (int e = threadIdx.x; e < F.E; e += kThreads) {
    int tot = 0;
    // eight blocks' masks in flight at a time (the loop is latency-bound)
#pragma unroll 8
    for (int b = 0; b < F.nb; ++b) tot += __popcll(F.bmask[(size_t)b * F.E + e]);
    scnt[e] = tot;
    stile[e] = cdiv(tot, F.BM);
    st_layout<COH>(F.counts + e, tot);
  }
  __syncthreads();
  const int R = block_exclusive_scan(scnt, F.E, tmp);
  const int ntiles = block_exclusive_scan(stile, F.E, tmp);
  const bool valid = R == F.R && ntiles <= F.max_tiles;
  if (!valid) {
    if (threadIdx.x == 0) {
      set_status(F.s.status, MOE_ERR_INVALID_ROUTE);
      st_layout<COH>(F.s.n_mtiles, 0);
    }
    for (int e = threadIdx.x; e <= F.E; e += kThreads) {
      st_layout<COH>(F.etile + e, 0);
      st_layout<COH>(F.offsets + e, 0);
    }
    return;
  }
  for (int e = threadIdx.x; e < F.E; e += kThreads) {
    const int off = scnt[e];
    st_layout<COH>(F.offsets + e, off);
    st_layout<COH>(F.etile + e, stile[e]);
    int run = off;
#pragma unroll 8
    for (int b = 0; b < F.nb; ++b) {
      st_layout<COH>(F.bbase + (size_t)b * F.E + e, run);
      run += __popcll(F.bmask[(size_t)b * F.E + e]);
    }
    const int cnt = run - off;
    for (int mt = 0, id = stile[e]; mt * F.BM < cnt; ++mt, ++id) {
      st_layout<COH>(F.tile_e + id, e);
      st_layout<COH>(F.tile_r0 + id, off + mt * F.BM);
      st_layout<COH>(F.tile_n + id, min(F.BM, cnt - mt * F.BM));
    }
  }
  if (threadIdx.x == 0) {
    st_layout<COH>(F.offsets + F.E, R);
    st_layout<COH>(F.etile + F.E, ntiles);
    st_layout<COH>(F.s.n_mtiles, ntiles);
  }
}

// Position of the rank-th set bit (0-based) of m.
__device__ __forceinline__ int select_bit(unsigned long long m, int rank) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const unsigned long long low = m & ((1ull << w) - 1ull);
    const int c = __popcll(low);
    if (rank >= c) {
      rank -= c;
      m >>= w;
      pos += w;
    } else {
      m = low;
    }
  }
  return pos;
}

// Source assignment of row r of expert e (rows in increasing assignment
// order): the block whose base is the last one <= r, then the matching set
// bit of that block's mask, then the slot of e among the token's experts.
__device__ __forceinline__ int row_source(const Fwd& F, int e, int r) {
  int lo = 0, hi = F.nb;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (F.bbase[(size_t)mid * F.E + e] <= r) lo = mid + 1; else hi = mid;
  }
  const int b = max(lo - 1, 0);
  const int rank = r - F.bbase[(size_t)b * F.E + e];
  const int t = min(b * kTokBlock + select_bit(F.bmask[(size_t)b * F.E + e], rank), F.T - 1);
  int j = 0;
  for (int jj = 0; jj < F.k; ++jj)
    if (F.topk[(size_t)t * F.k + jj] == e) j = jj;
  return t * F.k + j;
}

// Rows of one tile: writes perm, inv, the tile's source slot (and the
// per-row gate), then (if COPY) pulls the token rows into expert order.
// Raises ready[tile] (with the agent-scope release when REL: a reader runs
// in the same launch) unless the test-only MOE_FLAG_TEST_DROP_READY holds
// back the counter of row tile 0 (its readers' bounded waits then expire).
template <class Act, bool COPY, bool REL>
__device__ void gather_tile(const Fwd& F, int tile, int* ssrc) {
  const TileRows tr = fwd_tile(F, tile);
  const int e = tr.e, r0 = tr.r0, n = tr.n;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int r = r0 + i;
    const int a = row_source(F, e, r);
    const int t = a / F.k;
    F.perm[r] = a;
    F.inv[a] = r;
    F.tsrc[slots::tile_slot(tile, i, F.BM, 1)] = t;
    if (F.grow) F.grow[r] = F.gate[a];
    ssrc[i] = t;
  }
  __syncthreads();
  if (COPY) {
    const int wave = threadIdx.x >> 6;
    const int nvec = F.d * (int)sizeof(Act) / 16;
    const uint4* X = (const uint4*)F.x;
    uint4* XP = (uint4*)F.xp;
    for (int i = wave; i < n; i += 4)
      wave_copy_row(X + (size_t)ssrc[i] * nvec, XP + (size_t)(r0 + i) * nvec, nvec, CopyAsIs());
  }
  if (tile == 0 && (F.s.flags & MOE_FLAG_TEST_DROP_READY)) return;
  signal_add<REL>(&F.s.ready[tile], 1);
}

// ---------------------------------------------------------------- GEMMs
// CO: a reader of the tile's output runs in the same launch, so the output
// is stored coherently (kStoreCoherent) and published by signal_add_stored;
// otherwise ordinary stores (the kernel boundary publishes them).
template <class TL, bool CO>
__device__ void g1_tile_bf16(const Fwd& F, int tile, int nt, bf16_t* smem) {
  const TileRows tr = fwd_tile(F, tile);
  const int e = tr.e, r0 = tr.r0, n = tr.n;
  if (n <= 0) return;
  const int d = F.d, I = F.I;
  const bf16_t* W1 = (const bf16_t*)F.w1 + (size_t)e * I * d;
  const bf16_t* W3 = (const bf16_t*)F.w3 + (size_t)e * I * d;
  const int c0 = nt * (TL::BN / 2);
  typedef std::conditional_t<TL::kDMA, DmaRows<TL::BM, TL::KS>, KRows<TL::BM>> LA;
  typedef std::conditional_t<TL::kDMA, DmaRows<TL::BN, TL::KS>, KRows<TL::BN>> LB;
  LA la;
  LB lb;
  // rows past the tile's n repeat its last row (their outputs are dropped)
  if (F.direct) {
    const bf16_t* X = (const bf16_t*)F.x;
    const int* ts = F.tsrc + slots::tile_slot(tile, 0, F.BM, 1);
    la.init([&](int r) -> const bf16_t* { return X + (size_t)clamp_token(ts[min(r, n - 1)], F.T) * d; });
  } else {
    const bf16_t* XP = (const bf16_t*)F.xp;
    la.init([&](int r) -> const bf16_t* { return XP + (size_t)(r0 + min(r, n - 1)) * d; });
  }
  lb.init([&](int nr) -> const bf16_t* {
    int which, col;
    swiglu_brow<TL>(nr, which, col);
    return (which ? W3 : W1) + (size_t)(c0 + col) * d;
  });
  f32x16_t acc[TL::MI][TL::NJ];
  if constexpr (TL::kDMA)
    tile_mainloop_dma<TL>(d / TL::KS, smem, acc, la, lb);
  else
    tile_mainloop<TL>(d / 64, smem, acc, la, lb);
  // H (then the saved pre-activations) staged in LDS, stored 16 bytes a lane
  typedef Staged<TL::BM, TL::BN / 2> St;
  static_assert(St::bytes <= TL::smem_bytes, "SwiGLU staging fits the tile's LDS");
  bf16_t* H = (bf16_t*)F.h;
  bf16_t* A = (bf16_t*)F.a;
  bf16_t* B = (bf16_t*)F.b;
  const St st{smem};
  tile_visit_pairs<TL>(acc, [&](int row, int col, float av, float bv) { st.put(row, col, silu_f(av) * bv); });
  if constexpr (CO)
    st.flush_coherent(n, H + (size_t)r0 * I + c0, I);
  else
    st.flush(n, [&](int row) { return H + (size_t)(r0 + row) * I + c0; });
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

template <class TL, bool CO>
__device__ void g2_tile_bf16(const Fwd& F, int tile, int nt, bf16_t* smem) {
  const TileRows tr = fwd_tile(F, tile);
  const int e = tr.e, r0 = tr.r0, n = tr.n;
  if (n <= 0) return;
  const int d = F.d, I = F.I;
  const bf16_t* W2 = (const bf16_t*)F.w2 + (size_t)e * d * I;
  const bf16_t* H = (const bf16_t*)F.h;
  const int c0 = nt * TL::BN;
  static_assert(Staged<TL::BM, TL::BN>::bytes <= TL::smem_bytes, "output staging fits the tile's LDS");
  typedef std::conditional_t<TL::kDMA, DmaRows<TL::BM, TL::KS>, KRows<TL::BM>> LA;
  typedef std::conditional_t<TL::kDMA, DmaRows<TL::BN, TL::KS>, KRows<TL::BN>> LB;
  LA la;
  LB lb;
  la.init([&](int r) -> const bf16_t* { return H + (size_t)(r0 + min(r, n - 1)) * I; });
  lb.init([&](int nr) -> const bf16_t* { return W2 + (size_t)(c0 + nr) * I; });
  f32x16_t acc[TL::MI][TL::NJ];
  if constexpr (TL::kDMA)
    tile_mainloop_dma<TL>(I / TL::KS, smem, acc, la, lb);
  else
    tile_mainloop<TL>(I / 64, smem, acc, la, lb);
  bf16_t* YP = (bf16_t*)F.yp;
  const Staged<TL::BM, TL::BN> st{smem};
  tile_visit<TL>(acc, [&](int row, int col, float v) { st.put(row, col, v); });
  if constexpr (CO)
    st.flush_coherent(n, YP + (size_t)r0 * d + c0, d);
  else
    st.flush(n, [&](int row) { return YP + (size_t)(r0 + row) * d + c0; });
}

template <bool CO>
__device__ void g1_tile_f32(const Fwd& F, int tile, int nt, float* smem) {
  const TileRows tr = fwd_tile(F, tile);
  const int e = tr.e, r0 = tr.r0, n = tr.n;
  const int d = F.d, I = F.I;
  const float* W1 = (const float*)F.w1 + (size_t)e * I * d;
  const float* W3 = (const float*)F.w3 + (size_t)e * I * d;
  const float* XP = (const float*)F.xp;
  const int c0 = nt * 32;
  float acc[2][4];
  tile_f32(d, smem, acc,
           [&](int r) -> const float* { return r < n ? XP + (size_t)(r0 + r) * d : nullptr; },
           [&](int nr) -> const float* { return (nr < 32 ? W1 : W3) + (size_t)(c0 + (nr & 31)) * d; });
  float* H = (float*)F.h;
  float* A = (float*)F.a;
  float* B = (float*)F.b;
  tile_f32_visit_pairs(acc, [&](int row, int col, float av, float bv) {
    if (row < n) {
      const size_t o = (size_t)(r0 + row) * I + c0 + col;
      if constexpr (CO)  // an agent-coherent store (written through the L2)
        __hip_atomic_store(H + o, silu_f(av) * bv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        H[o] = silu_f(av) * bv;
      if (A) A[o] = av;
      if (B) B[o] = bv;
    }
  });
}

template <bool CO>
__device__ void g2_tile_f32(const Fwd& F, int tile, int nt, float* smem) {
  const TileRows tr = fwd_tile(F, tile);
  const int e = tr.e, r0 = tr.r0, n = tr.n;
  const int d = F.d, I = F.I;
  const float* W2 = (const float*)F.w2 + (size_t)e * d * I;
  const float* H = (const float*)F.h;
  const int c0 = nt * 64;
  float acc[2][4];
  tile_f32(I, smem, acc,
           [&](int r) -> const float* { return r < n ? H + (size_t)(r0 + r) * I : nullptr; },
           [&](int nr) -> const float* { return W2 + (size_t)(c0 + nr) * I; });
  float* YP = (float*)F.yp;
  tile_f32_visit(acc, [&](int row, int col, float v) {
    if (row >= n) return;
    if constexpr (CO)
      __hip_atomic_store(YP + (size_t)(r0 + row) * d + c0 + col, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      YP[(size_t)(r0 + row) * d + c0 + col] = v;
  });
}

// ---------------------------------------------------------------- combine
__device__ __forceinline__ Merge merge_of(const Fwd& F) { return Merge{F.T, F.d, F.k, F.R, F.yp, F.gate, F.inv, F.y}; }

// y[t] = sum_j gate[t,j] * yp[inv[t*k+j]], fp32 accumulation in slot order.
// K = k when known at compile time (every row load of a vector is issued
// before the first one is used), 0 for any k up to kMaxK.  COH: the merge
// runs in the launch whose gather tasks wrote inv; a 128-byte line of inv
// holds the slots of 4 tokens (k = 8), written by the gather tasks of
// several row tiles on any XCD, so an XCD whose L2 took the line in for its
// own partial write may hold stale bytes of the others: the indices are
// then read with coherent agent-scope loads.
template <class Act, int K, bool COH = false>
__device__ void combine_tokens_k(const Merge& F, int cb) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int EPV = 16 / sizeof(Act);  // elements per 16-byte vector
  constexpr int NR = K ? K : kMaxK;
  const int k = K ? K : F.k;
  const int nvec = F.d / EPV;
  for (int tt = wave; tt < kCombTok; tt += 4) {
    const int t = cb * kCombTok + tt;
    if (t >= F.T) break;
    int rows[NR];
    float g[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int* ip = F.inv + (size_t)t * k + j;
      rows[j] = j < k ? clamp_row(COH ? load_relaxed(ip) : *ip, F.R) : 0;
      g[j] = j < k ? F.gate[(size_t)t * k + j] : 0.0f;
    }
    // known k: kCombVec vectors per lane per step, every row load of a step
    // issued before the first is used, and the next step's loads issued
    // before this step's stores (vmcnt counts stores too: loads issued after
    // the stores would wait for them)
    constexpr int VU = K ? kCombVec : 1;
    if constexpr (K != 0) {
      uint4 u[VU][K], nx[VU][K];
      auto load = [&](uint4 (&b)[VU][K], int v) {
#pragma unroll
        for (int h = 0; h < VU; ++h)
#pragma unroll
          for (int j = 0; j < K; ++j)
            if (v + 64 * h < nvec) b[h][j] = ((const uint4*)F.yp)[(size_t)rows[j] * nvec + v + 64 * h];
      };
      load(u, lane);
      for (int v0 = lane; v0 < nvec; v0 += 64 * VU) {
        if (v0 + 64 * VU < nvec) load(nx, v0 + 64 * VU);
#pragma unroll
        for (int h = 0; h < VU; ++h) {
          if (v0 + 64 * h >= nvec) break;
          float acc[EPV];
#pragma unroll
          for (int q = 0; q < EPV; ++q) acc[q] = 0.0f;
#pragma unroll
          for (int j = 0; j < K; ++j) {
            const Act* p = (const Act*)&u[h][j];
#pragma unroll
            for (int q = 0; q < EPV; ++q) acc[q] = fmaf(g[j], Elem<Act>::to_f32(p[q]), acc[q]);
          }
          uint4 o;
          Act* po = (Act*)&o;
#pragma unroll
          for (int q = 0; q < EPV; ++q) po[q] = Elem<Act>::from_f32(acc[q]);
          ((uint4*)F.y)[(size_t)t * nvec + v0 + 64 * h] = o;
        }
#pragma unroll
        for (int h = 0; h < VU; ++h)
#pragma unroll
          for (int j = 0; j < K; ++j) u[h][j] = nx[h][j];
      }
    } else {
      for (int v = lane; v < nvec; v += 64) {
        float acc[EPV];
#pragma unroll
        for (int q = 0; q < EPV; ++q) acc[q] = 0.0f;
        for (int j = 0; j < k; ++j) {
          const uint4 u = ((const uint4*)F.yp)[(size_t)rows[j] * nvec + v];
          const Act* p = (const Act*)&u;
#pragma unroll
          for (int q = 0; q < EPV; ++q) acc[q] = fmaf(g[j], Elem<Act>::to_f32(p[q]), acc[q]);
        }
        uint4 o;
        Act* po = (Act*)&o;
#pragma unroll
        for (int q = 0; q < EPV; ++q) po[q] = Elem<Act>::from_f32(acc[q]);
        ((uint4*)F.y)[(size_t)t * nvec + v] = o;
      }
    }
  }
}

template <class Act, bool COH = false>
__device__ void combine_tokens(const Merge& F, int cb) {
  switch (F.k) {
    case 1: combine_tokens_k<Act, 1, COH>(F, cb); break;
    case 2: combine_tokens_k<Act, 2, COH>(F, cb); break;
    case 4: combine_tokens_k<Act, 4, COH>(F, cb); break;
    case 6: combine_tokens_k<Act, 6, COH>(F, cb); break;
    case 8: combine_tokens_k<Act, 8, COH>(F, cb); break;
    default: combine_tokens_k<Act, 0, COH>(F, cb); break;
  }
}

}  // namespace moe
