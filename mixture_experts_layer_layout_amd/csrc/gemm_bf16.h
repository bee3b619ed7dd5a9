// gemm_bf16.h -- one workgroup tile of a bf16 GEMM on CDNA4 matrix cores
// (v_mfma_f32_32x32x16_bf16, fp32 accumulate), used by every expert GEMM of
// the forward and backward.
//
// C[BM x BN] = sum_k A[m, k] * B[n, k], K consumed 64 at a time: two LDS
// stages and two register stages, so the global loads of two stages are in
// flight while a third feeds the MFMAs; one barrier per step.  LDS holds
// both operands k-contiguous: a row of 64 bf16 is 8 chunks of 16 bytes and
// chunk c of row r is stored at chunk c ^ lds_key(r) (lds_idx), so the
// 16-byte reads and writes of 16 lanes at a time hit 16 different bank
// groups.
//
// Operands come through loaders with three steps:
//   prep(kt)    addressing of stage kt (may itself load row indices); runs
//               one stage ahead of load() so those loads are in flight early
//   load(b, kt) the stage's global loads into register buffer b, all
//               unconditional
//               (no per-lane branches: padding rows are clamped to a
//               readable row, or aimed at a zero row when they must add 0)
//   store(b, lds) register buffer b into LDS; any scaling happens here, after
//               the MFMAs of the previous stage, so no load result is
//               consumed early
// Loader kinds:
//   KRows   the operand is stored as rows with k contiguous (row-major
//           [rows, K]); rows may be gathered through an index (pull)
//   KCols   the operand is stored with k as the row index and the tile's
//           rows contiguous ([K, rows]); each thread loads a KK x 8 block
//           and transposes it in registers before the LDS store
// Four waves split the tile 2 x 2; each wave owns (BM/2) x (BN/2) in
// (BM/64) x (BN/64) MFMA blocks of 32 x 32.
#pragma once

#include "common.h"

namespace moe {

// The XOR key of tile row `row`: chunk c of the row is stored at slot
// c ^ key.  (row >> 1) & 7 places the same chunk of 16 aligned consecutive
// rows in distinct slot pairs and the 8 chunks of one row in 8 slots, which
// the fragment reads (32 consecutive rows, one chunk) and the row-wise
// 16-byte stores need; the K-major loader's 8-byte stores (a lane group
// writes rows 8 apart, one per column block) also need column blocks of
// equal parity apart.  HI XORs in row >> 4 for that.  Measured per access
// pattern with single-pattern probe kernels (SQ_LDS_BANK_CONFLICT over
// SQ_LDS_IDX_ACTIVE): with HI the fragment reads, the row stores and the
// K-major stores (4 or 8 k-rows a thread) all run without conflicts, 4 LDS
// cycles per fragment read and per 8-byte store instruction.  The plain key
// has the K-major stores at 16 cycles (75% conflict cycles); the earlier
// term (row >> 4) << 1 had both the fragment reads and those stores at 8.
// The direct-to-LDS forward tile keeps the plain key (TileD::kKeyHi): its
// fragment reads and DMA writes are conflict-free with it and it has no
// K-major stores.
template <bool HI>
__device__ __forceinline__ int lds_key(int row) {
  return HI ? ((row >> 1) ^ (row >> 4)) & 7 : (row >> 1) & 7;
}

// Element index of 16-byte chunk `chunk` of tile row `row` in an LDS stage.
template <bool HI>
__device__ __forceinline__ int lds_idx(int row, int chunk) {
  return (row << 6) + ((chunk ^ lds_key<HI>(row)) << 3);
}

// The same for a stage of KS k values a row: 64 (the layout above) or 32
// (64-byte rows, four chunks; the key (row >> 2) & 3 puts the 16-byte
// reads of 8 consecutive rows in 8 distinct groups of four banks: rows
// 4 apart sit 256 bytes apart, and the key moves rows 4..7 of a group of
// 8 to the other chunk of a pair).
template <int KS, bool HI>
__device__ __forceinline__ int stage_key(int row) {
  static_assert(KS == 64 || (KS == 32 && !HI), "64-k stages (either key) or 32-k stages (plain key)");
  if constexpr (KS == 64)
    return lds_key<HI>(row);
  else
    return (row >> 2) & 3;
}
template <int KS, bool HI>
__device__ __forceinline__ int stage_idx(int row, int chunk) {
  return row * KS + ((chunk ^ stage_key<KS, HI>(row)) << 3);
}

// Stages whose global loads are in flight while one stage feeds the MFMAs
// (register buffers per loader).  Measured: 2 gave no gain over 1 on the
// expert GEMMs, and its 32 extra VGPRs keep the persistent kernels from
// fitting two workgroups per CU.
#ifndef MOE_PREFETCH
#define MOE_PREFETCH 1
#endif
constexpr int kPrefetch = MOE_PREFETCH;
static_assert(kPrefetch == 1 || kPrefetch == 2, "prefetch distance 1 or 2");

// A tile shape and its operand type.  LDS_A / LDS_B are the sizes of one
// stage of each operand in bf16 units; stage() runs the MFMAs of one stage
// held in LDS (the main loop below is shared by every tile type).
template <int BM_, int BN_>
struct Tile {
  static constexpr bool kMX = false;
  static constexpr bool kDMA = false;
  static constexpr bool kKeyHi = true;  // lds_key<true>
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int MI = WM / 32, NJ = WN / 32;
  static constexpr int KS = 64;  // k values per stage
  static constexpr int LDS_A = BM * 64, LDS_B = BN * 64;
  static constexpr size_t smem_bytes = 2 * (LDS_A + LDS_B) * sizeof(bf16_t);
  static __device__ __forceinline__ void stage(const bf16_t* As, const bf16_t* Bs, f32x16_t (&acc)[MI][NJ]);
};

// ---------------------------------------------------------------- loaders
// Rows with k contiguous.  Thread t handles chunk t%8 of rows t/8 + 32*i.
template <int ROWS, int NBUF = kPrefetch>
struct KRows {
  static constexpr int PER = ROWS / 32;
  const bf16_t* row[PER];
  uint4 v[NBUF][PER];
  // rowptr(r) -> pointer to element k=0 of tile row r; must be readable
  // for every r (clamp rows past the operand to a real one).
  template <class F>
  __device__ __forceinline__ void init(F rowptr) {
    const int r0 = threadIdx.x >> 3;
#pragma unroll
    for (int i = 0; i < PER; ++i) row[i] = rowptr(r0 + 32 * i);
  }
  __device__ __forceinline__ void prep(int) {}
  template <int BUF>
  __device__ __forceinline__ void load(int kt) {
    const int ch = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < PER; ++i) v[BUF][i] = *(const uint4*)(row[i] + kt * 64 + ch * 8);
  }
  template <int BUF, bool HI>
  __device__ __forceinline__ void store(bf16_t* lds) const {
    const int r0 = threadIdx.x >> 3, ch = threadIdx.x & 7;
#pragma unroll
    for (int i = 0; i < PER; ++i) *(uint4*)(lds + lds_idx<HI>(r0 + 32 * i, ch)) = v[BUF][i];
  }
};

// k is the row index of the stored operand; the tile's ROWS rows are
// contiguous within each stored row.  Each thread covers one k-group (KK
// consecutive k) and 8 tile rows (kgroup(), cblock()), with KK = 8 for
// 256-row tiles and 4 for 128-row tiles, so all 256 threads take part.
//   kptr(k, c) pointer to the stored row holding k, at the tile's first
//             row; never null (k past the operand -> a zero row).  c is the
//             column tile of a stream (tile_stream), 0 otherwise
//   kscale(k) factor for that stored row (SCALED only)
//   half_off  extra element offset for the second half of the tile's rows
//             (two column ranges of one stored row, e.g. the dA and dB
//             halves of [dA | dB]); 0 when the rows are contiguous
template <int ROWS, bool SCALED, class P, class S, int NBUF = kPrefetch>
struct KCols {
  static constexpr int KK = ROWS >= 256 ? 8 : 4;
  static constexpr int KG = 64 / KK;
  static_assert(KG * (ROWS / 8) == kThreads, "KCols covers the stage with every thread");
  P kptr;
  S kscale;
  int coff;
  int nk_ = 0;  // stages per column tile when streamed (tile_stream), else 0
  // position of the last prepared step: step pj_ = column tile pc_, stage
  // ps_ (prep is called with steps that grow by 0 or 1 at a time)
  int pj_ = -1, pc_ = 0, ps_ = -1;
  const bf16_t* p[KK];
  float s[KK], sl[NBUF][KK];
  uint4 v[NBUF][KK];
  // thread -> (k-group, 8-column block), so that every load instruction of
  // a wave reads whole 128-byte lines: 8 k-rows x 8 column blocks.  With
  // KG = 16 (128-row tiles) wave w takes k-groups 8 (w >> 1) .. +7 and
  // column blocks 8 (w & 1) .. +7 (the split t % KG, t / KG read 16 k-rows x
  // 64 bytes a wave, half lines: the backward took 17.25 ms against 16.16
  // ms at the DeepSeek-V3 Zipf shape); with KG = 8 that split already
  // reads 8 k-rows x 128 bytes.
  __device__ static __forceinline__ int kgroup() {
    if (KG == 16) return 8 * (threadIdx.x >> 7) + ((threadIdx.x & 63) >> 3);
    return threadIdx.x % KG;
  }
  __device__ static __forceinline__ int cblock() {
    if (KG == 16) return 8 * ((threadIdx.x >> 6) & 1) + (threadIdx.x & 7);
    return threadIdx.x / KG;
  }
  __device__ __forceinline__ KCols(P kp, S ks, int half_off) : kptr(kp), kscale(ks) {
    const int nb = cblock();
    coff = nb * 8 + (nb >= ROWS / 16 ? half_off : 0);
  }
  __device__ __forceinline__ void prep(int kt) {
    if (nk_ == 0) {
      pc_ = 0;
      ps_ = kt;
    } else if (kt == pj_ + 1) {
      if (++ps_ == nk_) {
        ps_ = 0;
        ++pc_;
      }
    } else if (kt != pj_) {
      pc_ = kt / nk_;
      ps_ = kt - pc_ * nk_;
    }
    pj_ = kt;
    const int c = pc_;
    const int k0 = ps_ * 64 + kgroup() * KK;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      p[kk] = kptr(k0 + kk, c);
      if (SCALED) s[kk] = kscale(k0 + kk);
    }
  }
  template <int BUF>
  __device__ __forceinline__ void load(int) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      v[BUF][kk] = *(const uint4*)(p[kk] + coff);
      if (SCALED) sl[BUF][kk] = s[kk];
    }
  }
  template <int BUF, bool HI>
  __device__ __forceinline__ void store(bf16_t* lds) {
    uint32_t* w = (uint32_t*)v[BUF];  // w[kk*4 + q] = elements 2q, 2q+1 of k-row kk
    if (SCALED) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          w[kk * 4 + q] = pack_bf16x2(bf16_to_f32((bf16_t)(w[kk * 4 + q] & 0xffff)) * sl[BUF][kk],
                                      bf16_to_f32((bf16_t)(w[kk * 4 + q] >> 16)) * sl[BUF][kk]);
    }
    const int kg = kgroup(), nb = cblock();
    // lanes of odd nb walk their 8 rows in the order 1,0,3,2,...: the two
    // lane groups written together then target rows of opposite parity,
    // i.e. opposite halves of the 256-byte bank row
    const int odd = nb & 1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int mm = i ^ odd;
      // element mm of each k-row: dword mm/2 (= i/2), half mm%2
      const int q = i >> 1;
      const uint32_t sel = (mm & 1) ? 0x07060302u : 0x05040100u;
      if (KK == 8) {
        uint4 o;
        o.x = __builtin_amdgcn_perm(w[1 * 4 + q], w[0 * 4 + q], sel);
        o.y = __builtin_amdgcn_perm(w[3 * 4 + q], w[2 * 4 + q], sel);
        o.z = __builtin_amdgcn_perm(w[5 * 4 + q], w[4 * 4 + q], sel);
        o.w = __builtin_amdgcn_perm(w[7 * 4 + q], w[6 * 4 + q], sel);
        *(uint4*)(lds + lds_idx<HI>(nb * 8 + mm, kg)) = o;
      } else {
        uint2 o;
        o.x = __builtin_amdgcn_perm(w[1 * 4 + q], w[0 * 4 + q], sel);
        o.y = __builtin_amdgcn_perm(w[3 * 4 + q], w[2 * 4 + q], sel);
        *(uint2*)(lds + lds_idx<HI>(nb * 8 + mm, kg >> 1) + (kg & 1) * 4) = o;
      }
    }
  }
};

struct NoScale {
  __device__ __forceinline__ float operator()(int) const { return 1.0f; }
};

template <int ROWS, class P>
__device__ __forceinline__ KCols<ROWS, false, P, NoScale> kcols(P kptr, int half_off = 0) {
  return KCols<ROWS, false, P, NoScale>(kptr, NoScale(), half_off);
}
// the same with NBUF register buffers (a deeper prefetch; tile_band's
// streamed operand)
template <int ROWS, int NBUF, class P>
__device__ __forceinline__ KCols<ROWS, false, P, NoScale, NBUF> kcols_n(P kptr, int half_off = 0) {
  return KCols<ROWS, false, P, NoScale, NBUF>(kptr, NoScale(), half_off);
}
template <int ROWS, class P, class S>
__device__ __forceinline__ KCols<ROWS, true, P, S> kcols_scaled(P kptr, S kscale, int half_off = 0) {
  return KCols<ROWS, true, P, S>(kptr, kscale, half_off);
}

// ---------------------------------------------------------------- core
// The 64-deep stage as 4 k-slices of 16; the operand fragments of slice
// s+1 are read from LDS before the MFMAs of slice s are issued, so the LDS
// latency hides behind them.
template <class TL>
__device__ __forceinline__ void tile_compute(const bf16_t* As, const bf16_t* Bs,
                                             f32x16_t (&acc)[TL::MI][TL::NJ]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int NKS = TL::KS / 16;  // MFMA k-slices per stage
  bf16x8_t a[2][TL::MI], b[2][TL::NJ];
  auto frags = [&](int ks, bf16x8_t(&fa)[TL::MI], bf16x8_t(&fb)[TL::NJ]) {
    const int ch = ks * 2 + (lane >> 5);
#pragma unroll
    for (int i = 0; i < TL::MI; ++i)
      fa[i] = *(const bf16x8_t*)(As + stage_idx<TL::KS, TL::kKeyHi>(wm * TL::WM + 32 * i + (lane & 31), ch));
#pragma unroll
    for (int j = 0; j < TL::NJ; ++j)
      fb[j] = *(const bf16x8_t*)(Bs + stage_idx<TL::KS, TL::kKeyHi>(wn * TL::WN + 32 * j + (lane & 31), ch));
  };
  frags(0, a[0], b[0]);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (ks < NKS - 1) frags(ks + 1, a[(ks + 1) & 1], b[(ks + 1) & 1]);
#pragma unroll
    for (int i = 0; i < TL::MI; ++i)
#pragma unroll
      for (int j = 0; j < TL::NJ; ++j) acc[i][j] = mfma32x32x16(a[ks & 1][i], b[ks & 1][j], acc[i][j]);
  }
  // instruction order for the scheduler: the reads of slice 0, then per
  // slice the reads of the next slice ahead of this slice's MFMAs
  constexpr int NR = TL::MI + TL::NJ, NM = TL::MI * TL::NJ;
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (ks < NKS - 1) __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
  }
}

template <int BM_, int BN_>
__device__ __forceinline__ void Tile<BM_, BN_>::stage(const bf16_t* As, const bf16_t* Bs, f32x16_t (&acc)[MI][NJ]) {
  tile_compute<Tile<BM_, BN_>>(As, Bs, acc);
}

// Runs the K loop over nk stages (nk may be 0: the tile is then zero).
// PF stages are in flight in registers while a third feeds the MFMAs from
// LDS: at step kt the loads of stage kt+PF go into register buffer kt % PF
// (stored to LDS a step earlier), the MFMAs consume stage kt from LDS
// buffer kt % 2, and stage kt+1 (register buffer (kt+1) % PF) is written to
// the other LDS buffer.  Every load, prep and store is unconditional --
// past the last stage they repeat it -- so the only waits the compiler
// emits are for the stage being stored.  STEP is kt modulo lcm(2, PF), so
// both buffer indices are compile-time.
template <int STEP, class TL, int PF = kPrefetch, class LA, class LB>
__device__ __forceinline__ void mainloop_step(int kt, int last, bf16_t* As, bf16_t* Bs,
                                              f32x16_t (&acc)[TL::MI][TL::NJ], LA& A, LB& B) {
  constexpr int CUR = STEP & 1;            // LDS buffer read now
  constexpr int RB = STEP % PF;            // register buffer loaded now
  constexpr int SB = (STEP + 1) % PF;      // register buffer stored now
  A.template load<RB>(min(kt + PF, last));
  B.template load<RB>(min(kt + PF, last));
  A.prep(min(kt + PF + 1, last));
  B.prep(min(kt + PF + 1, last));
  // keep the scheduler from sinking these loads below the LDS stores of
  // the previous stage (which wait for their own loads)
  __builtin_amdgcn_sched_barrier(0);
  TL::stage(As + CUR * TL::LDS_A, Bs + CUR * TL::LDS_B, acc);
  __builtin_amdgcn_sched_barrier(0);
  A.template store<SB, TL::kKeyHi>(As + (CUR ^ 1) * TL::LDS_A);
  B.template store<SB, TL::kKeyHi>(Bs + (CUR ^ 1) * TL::LDS_B);
  __syncthreads();
}

// Loads the first PF stages (stage s into register buffer s) and stores
// stage 0 into LDS buffer 0.
template <class TL, int PF = kPrefetch, class LA, class LB>
__device__ __forceinline__ void mainloop_prologue(int last, bf16_t* As, bf16_t* Bs, LA& A, LB& B) {
  A.prep(0);
  B.prep(0);
  A.template load<0>(0);
  B.template load<0>(0);
  A.prep(min(1, last));
  B.prep(min(1, last));
  if constexpr (PF >= 2) {
    A.template load<1>(min(1, last));
    B.template load<1>(min(1, last));
    A.prep(min(2, last));
    B.prep(min(2, last));
  }
  if constexpr (PF >= 3) {
    A.template load<2>(min(2, last));
    B.template load<2>(min(2, last));
    A.prep(min(3, last));
    B.prep(min(3, last));
  }
  if constexpr (PF >= 4) {
    A.template load<3>(min(3, last));
    B.template load<3>(min(3, last));
    A.prep(min(4, last));
    B.prep(min(4, last));
  }
  __syncthreads();
  A.template store<0, TL::kKeyHi>(As);
  B.template store<0, TL::kKeyHi>(Bs);
  __syncthreads();
}

// Steps STEP .. U-1 of one unrolled round of U steps, each only if its
// stage exists.
template <int STEP, int U, class TL, int PF, class LA, class LB>
__device__ __forceinline__ void mainloop_tail(int kt, int nk, int last, bf16_t* As, bf16_t* Bs,
                                              f32x16_t (&acc)[TL::MI][TL::NJ], LA& A, LB& B) {
  if constexpr (STEP < U) {
    if (kt + STEP < nk) {
      mainloop_step<STEP, TL, PF>(kt + STEP, last, As, Bs, acc, A, B);
      mainloop_tail<STEP + 1, U, TL, PF>(kt, nk, last, As, Bs, acc, A, B);
    }
  }
}

template <int STEP, int U, class TL, int PF, class LA, class LB>
__device__ __forceinline__ void mainloop_round(int kt, int last, bf16_t* As, bf16_t* Bs,
                                               f32x16_t (&acc)[TL::MI][TL::NJ], LA& A, LB& B) {
  if constexpr (STEP < U) {
    mainloop_step<STEP, TL, PF>(kt + STEP, last, As, Bs, acc, A, B);
    mainloop_round<STEP + 1, U, TL, PF>(kt, last, As, Bs, acc, A, B);
  }
}

// PF: stages loaded ahead into registers, 1 to 4 (the loaders need PF
// buffers).
template <class TL, int PF = kPrefetch, class LA, class LB>
__device__ __forceinline__ void tile_mainloop(int nk, bf16_t* smem, f32x16_t (&acc)[TL::MI][TL::NJ], LA& A,
                                              LB& B) {
  static_assert(PF >= 1 && PF <= 4, "register prefetch depth 1..4");
  constexpr int U = PF % 2 ? 2 * PF : PF;  // lcm(2, PF)
#pragma unroll
  for (int i = 0; i < TL::MI; ++i)
#pragma unroll
    for (int j = 0; j < TL::NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  if (nk <= 0) return;
  const int last = nk - 1;
  bf16_t* As = smem;
  bf16_t* Bs = smem + 2 * TL::LDS_A;
  mainloop_prologue<TL, PF>(last, As, Bs, A, B);
  int kt = 0;
  for (; kt + U <= nk; kt += U) mainloop_round<0, U, TL, PF>(kt, last, As, Bs, acc, A, B);
  mainloop_tail<0, U, TL, PF>(kt, nk, last, As, Bs, acc, A, B);
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

// ---------------------------------------------------------------- stream
// nc output tiles that share their A rows, each over nk K-stages, run as one
// stream of nc * nk steps (step j = column tile c = j / nk, stage s =
// j % nk, both advanced without division): the register prefetch runs
// across tile boundaries, so the next tile's loads overlap this tile's
// MFMAs and stores.  After the last stage of column tile c, epi(c, acc)
// writes the tile and the accumulators restart from zero.  The loaders'
// prep(j) must map the step to (c, stage) (KCols::nk_).
template <int CUR, class TL, class LA, class LB, class EPI>
__device__ __forceinline__ void stream_step(int j, int s, int c, int nk, int last, bf16_t* As, bf16_t* Bs,
                                            f32x16_t (&acc)[TL::MI][TL::NJ], LA& A, LB& B, EPI& epi) {
  constexpr int RB = kPrefetch == 2 ? CUR : 0;
  constexpr int SB = kPrefetch == 2 ? (CUR ^ 1) : 0;
  A.template load<RB>(min(j + kPrefetch, last));
  B.template load<RB>(min(j + kPrefetch, last));
  A.prep(min(j + kPrefetch + 1, last));
  B.prep(min(j + kPrefetch + 1, last));
  __builtin_amdgcn_sched_barrier(0);
  TL::stage(As + CUR * TL::LDS_A, Bs + CUR * TL::LDS_B, acc);
  __builtin_amdgcn_sched_barrier(0);
  A.template store<SB, TL::kKeyHi>(As + (CUR ^ 1) * TL::LDS_A);
  B.template store<SB, TL::kKeyHi>(Bs + (CUR ^ 1) * TL::LDS_B);
  if (s == nk - 1) {
    epi(c, acc);
#pragma unroll
    for (int i = 0; i < TL::MI; ++i)
#pragma unroll
      for (int jj = 0; jj < TL::NJ; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;
  }
  __syncthreads();
}

template <class TL, class LA, class LB, class EPI>
__device__ __forceinline__ void tile_stream(int nc, int nk, bf16_t* smem, LA& A, LB& B, EPI epi) {
  static_assert(!TL::kMX, "bf16 tiles");
  f32x16_t acc[TL::MI][TL::NJ];
#pragma unroll
  for (int i = 0; i < TL::MI; ++i)
#pragma unroll
    for (int j = 0; j < TL::NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const int total = nc * nk;
  if (total <= 0) return;
  const int last = total - 1;
  bf16_t* As = smem;
  bf16_t* Bs = smem + 2 * TL::LDS_A;
  mainloop_prologue<TL>(last, As, Bs, A, B);
  int j = 0, s = 0, c = 0;
  auto advance = [&] {
    if (++s == nk) {
      s = 0;
      ++c;
    }
  };
  for (; j + 1 < total; j += 2) {
    stream_step<0, TL>(j, s, c, nk, last, As, Bs, acc, A, B, epi);
    advance();
    stream_step<1, TL>(j + 1, s, c, nk, last, As, Bs, acc, A, B, epi);
    advance();
  }
  if (j < total) stream_step<0, TL>(j, s, c, nk, last, As, Bs, acc, A, B, epi);
}

// ---------------------------------------------------------------- band
// The nc output tiles of a band that share their A rows, when K is only
// NK = 1 or 2 stages (the weight gradients of experts with at most 128
// rows): A is loaded into LDS once and stays there, and only B streams,
// two stages ahead in registers.  Each tile's output is written at the end
// of its last stage.
//
// The point is the order of memory operations.  vmcnt counts loads and
// stores together, in issue order, so waiting for a load also waits for
// every store issued before it.  Here the B stage stored to LDS in step j
// was loaded at the top of step j-1, before that step's output stores, so
// the wait for it leaves those stores in flight; they have until the wait
// of step j+1 to complete.  For the compiler to count this exactly, every
// path into a step must have issued the same operations: the epilogue sits
// at a fixed place in the unrolled loop, and the steps before the repeating
// pattern (one step for NK = 1, one tile for NK = 2) are peeled.
template <int CUR, int S, bool EPI_NOW, class TL, class LB, class EPI>
__device__ __forceinline__ void band_step(int j, int c, int last, const bf16_t* As, bf16_t* Bs,
                                          f32x16_t (&acc)[TL::MI][TL::NJ], LB& B, EPI& epi) {
  B.template load<CUR>(min(j + 2, last));
  B.prep(min(j + 3, last));
  __builtin_amdgcn_sched_barrier(0);
  TL::stage(As + S * TL::LDS_A, Bs + CUR * TL::LDS_B, acc);
  __builtin_amdgcn_sched_barrier(0);
  B.template store<CUR ^ 1, TL::kKeyHi>(Bs + (CUR ^ 1) * TL::LDS_B);
  if (EPI_NOW) {
    epi(c, acc);
#pragma unroll
    for (int i = 0; i < TL::MI; ++i)
#pragma unroll
      for (int jj = 0; jj < TL::NJ; ++jj)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][jj][r] = 0.0f;
  }
  __syncthreads();
}

// A: the loader of the shared rows (prep(s) with s < NK gives stage s);
// B: a two-buffer loader (kcols_n<.., 2>) whose prep(j) maps step j to column tile
// j / NK, stage j % NK.  LDS: NK stages of A, then two B stages.
template <class TL, int NK, class LA, class LB, class EPI>
__device__ __forceinline__ void tile_band(int nc, bf16_t* smem, LA& A, LB& B, EPI epi) {
  static_assert(!TL::kMX && !TL::kDMA, "register-staged bf16 tiles");
  static_assert(NK == 1 || NK == 2, "one or two resident stages");
  static_assert((size_t)(NK * TL::LDS_A + 2 * TL::LDS_B) * sizeof(bf16_t) <= TL::smem_bytes, "band fits the LDS");
  f32x16_t acc[TL::MI][TL::NJ];
#pragma unroll
  for (int i = 0; i < TL::MI; ++i)
#pragma unroll
    for (int j = 0; j < TL::NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const int total = nc * NK;
  if (total <= 0) return;
  const int last = total - 1;
  bf16_t* As = smem;
  bf16_t* Bs = smem + NK * TL::LDS_A;
  // the LDS may still be read by the previous user
  __syncthreads();
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    A.prep(s);
    A.template load<0>(s);
    A.template store<0, TL::kKeyHi>(As + s * TL::LDS_A);
  }
  B.prep(0);
  B.template load<0>(0);
  B.prep(min(1, last));
  B.template load<1>(min(1, last));
  B.prep(min(2, last));
  B.template store<0, TL::kKeyHi>(Bs);
  __syncthreads();
  if (NK == 1) {
    band_step<0, 0, true, TL>(0, 0, last, As, Bs, acc, B, epi);
    int j = 1;
    for (; j + 1 < total; j += 2) {
      band_step<1, 0, true, TL>(j, j, last, As, Bs, acc, B, epi);
      band_step<0, 0, true, TL>(j + 1, j + 1, last, As, Bs, acc, B, epi);
    }
    if (j < total) band_step<1, 0, true, TL>(j, j, last, As, Bs, acc, B, epi);
  } else {
    band_step<0, 0, false, TL>(0, 0, last, As, Bs, acc, B, epi);
    band_step<1, 1, true, TL>(1, 0, last, As, Bs, acc, B, epi);
    for (int c = 1; c < nc; ++c) {
      band_step<0, 0, false, TL>(2 * c, c, last, As, Bs, acc, B, epi);
      band_step<1, 1, true, TL>(2 * c + 1, c, last, As, Bs, acc, B, epi);
    }
  }
}

// Writes a tile whose rows are all valid as bf16 with 16-byte stores, each
// covering 8 rows x 128 contiguous bytes (one wave's 64 columns).  The
// accumulators hold one column per lane, so each wave regroups its 64 x 64
// block through its own 2 KB of LDS (stage: 4 waves x 2 KB, used by no one
// else, so no barrier), 16 rows at a time: lane pairs swap values (DPP) so
// the even lane of a pair holds two columns of row r and the odd lane the
// same two columns of row r+1, each lane writes those words, and reads back
// 16-byte row chunks.  Four times fewer store instructions than storing
// the word pairs directly, whose 64 addresses per instruction kept the
// texture unit's address queue full.  The stores are buffer stores (the
// wave's base in a scalar descriptor, row offsets in scalar registers, one
// VGPR of lane offset).  Wave row block wm (tile rows wm * WM ..) starts at
// base(wm), rows ld elements apart; 128 * ld * 2 bytes stay below 2^31.
// LDS layout of a wave's 16 x 64 block: 32 dwords a row, the row's 16-byte
// chunk c at c ^ (4 * ((row >> 2) & 1)): conflict-free for the word writes
// (rows r, r+1, r+4, r+5 together) and the chunk reads (8 lanes a row).
constexpr int kWgradStageBytes = 4 * 2048;
// The weight-gradient stores carry the non-temporal hint (cache policy
// bit 1): 22.5 GB of dW written once at the DeepSeek-V3 shape would
// otherwise displace the band's inputs from the L2, and the data gradient
// the next launch reads.  Measured: dW1/dW3 5.66 -> 5.48 ms, the dX
// gather-sum after them 156 -> 109 us.
constexpr int kWgradStorePolicy = 2;
template <class TL, class BASE>
__device__ __forceinline__ void tile_store_staged(const f32x16_t (&acc)[TL::MI][TL::NJ], BASE base, size_t ld,
                                                  bf16_t* stage) {
  static_assert(TL::WN == 64 && TL::NJ == 2 && TL::WM == 32 * TL::MI, "64-column wave blocks");
  typedef unsigned int u32x4_t __attribute__((__vector_size__(16)));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int odd = lane & 1;
  uint32_t* st = (uint32_t*)stage + wave * 512;
  auto sidx = [](int row, int dw) { return row * 32 + ((((dw >> 2) ^ (((row >> 2) & 1) << 2)) << 2) | (dw & 3)); };
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(wave_uniform(base(wm)));
  const int ldb = (int)ld * 2;
  const int rrow = lane >> 3, rch = lane & 7;
  const int vo = rrow * ldb + (wn * TL::WN + 8 * rch) * 2;
#pragma unroll
  for (int i = 0; i < TL::MI; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // accumulator entries 8h .. 8h+7: rows 16h .. 16h+15 of block i
#pragma unroll
      for (int r = 8 * h; r < 8 * h + 8; r += 2) {
        const int row = 8 * ((r >> 2) & 1) + 4 * (lane >> 5) + (r & 3) + odd;
#pragma unroll
        for (int j = 0; j < TL::NJ; ++j) {
          const float v0 = acc[i][j][r], v1 = acc[i][j][r + 1];
          const float o0 = swap_lane_pair(v0), o1 = swap_lane_pair(v1);
          st[sidx(row, 16 * j + ((lane & 30) >> 1))] = odd ? pack_bf16x2(o1, v1) : pack_bf16x2(v0, o0);
        }
      }
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const u32x4_t q = *(const u32x4_t*)(st + sidx(8 * g + rrow, 4 * rch));
        __builtin_amdgcn_raw_buffer_store_b128(q, rs, vo, (32 * i + 16 * h + 8 * g) * ldb, kWgradStorePolicy);
        store_data_guard();
      }
    }
}

// ---------------------------------------------------------------- epilogue
// A [ROWS x W] bf16 block staged in LDS, then written out with 16-byte
// stores: block row r (r < nrows) goes to dst(r), a pointer to the block's
// first column in that output row.  The LDS row pitch is padded by 16 bytes
// so the 2-byte writes of the MFMA accumulator layout spread over the banks.
// The caller synchronises before reusing the LDS after flush().
template <int ROWS, int W>
struct Staged {
  static constexpr int LD = W + 8;
  static constexpr size_t bytes = (size_t)ROWS * LD * sizeof(bf16_t);
  bf16_t* s;
  __device__ __forceinline__ void put(int row, int col, float v) const { s[row * LD + col] = f32_to_bf16(v); }
  template <class D>
  __device__ __forceinline__ void flush(int nrows, D dst) const {
    __syncthreads();
    constexpr int CPR = W / 8;
    for (int c = threadIdx.x; c < ROWS * CPR; c += kThreads) {
      const int row = c / CPR, ch = c % CPR;
      if (row < nrows) *(uint4*)(dst(row) + ch * 8) = *(const uint4*)(s + row * LD + ch * 8);
    }
  }
  // The same block written coherently (kStoreCoherent) to rows `ld`
  // elements apart from `base` (the block's first element of its first
  // row; the block spans less than 2^31 bytes), for a reader in the same
  // launch (signal_add_stored).
  __device__ __forceinline__ void flush_coherent(int nrows, bf16_t* base, size_t ld) const {
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(wave_uniform(base));
    constexpr int CPR = W / 8;
    for (int c = threadIdx.x; c < ROWS * CPR; c += kThreads) {
      const int row = c / CPR, ch = c % CPR;
      if (row < nrows)
        store_coherent(rs, (int)(((size_t)row * ld + ch * 8) * sizeof(bf16_t)), *(const uint4*)(s + row * LD + ch * 8));
    }
  }
};

// Map a B-tile row of the SwiGLU tile to (which, out_col): which 0 = W1,
// 1 = W3; out_col in [0, BN/2).
template <class TL>
__device__ __forceinline__ void swiglu_brow(int n, int& which, int& col) {
  const int wn = n / TL::WN, w = n % TL::WN;
  which = w / (TL::WN / 2);
  col = wn * (TL::WN / 2) + (w % (TL::WN / 2));
}

}  // namespace moe
