// moe.hip -- kernels and C-ABI entry points of libmoe.so (gfx950).
//
// The forward and the backward each run either as one persistent kernel
// (desc->fused = 1) whose workgroups claim tasks phase by phase from
// per-XCD queues and wait on the device counters of their inputs, or as one
// kernel per step on the caller's stream.  Both call the same task
// functions (tasks_fwd.h, tasks_bwd.h).  A task waits only on tasks of
// earlier phases, all of which were claimed by running workgroups before it
// (sched.h); so the queues drain whatever the grid size, and every wait is
// additionally bounded (MOE_ERR_TIMEOUT) so a fault cannot hang them.
#include <hip/hip_runtime.h>

#include <string.h>

#include <mutex>
#include <type_traits>

#include "plan.h"
#include "tasks_fwd.h"
#include "tasks_bwd.h"
#include "sched.h"
#include "mxfp8.h"
#include "router_bwd.h"
#include "bwd_mx.h"

namespace moe {

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int make_plan(const moe_desc* D, Plan* p, bool fwd_only) {
  if (!D || !p) return MOE_ERR_INVALID_ARG;
  memset(p, 0, sizeof(*p));
  if (D->T < 0 || D->macro_tokens < 0) return MOE_ERR_INVALID_ARG;
  const bool macro = D->macro_tokens > 0 && D->macro_tokens < D->T;
  // macrobatches run the forward only, through a ring of two slots
  if (macro) fwd_only = true;
  // with macrobatches every size below is that of one macrobatch
  const int T = macro ? D->macro_tokens : D->T, d = D->d, E = D->E, k = D->k, I = D->I;
  if (d <= 0 || E <= 0 || k <= 0 || I <= 0) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE || k > kMaxK || k > E) return MOE_ERR_INVALID_ARG;
  if ((int64_t)T * k > (int64_t)1 << 30) return MOE_ERR_INVALID_ARG;
  if (D->score != MOE_SCORE_SOFTMAX && D->score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  const bool f32 = D->act_dtype == MOE_F32;
  if (f32) {
    if (D->expert_dtype != MOE_F32) return MOE_ERR_UNSUPPORTED;
    if (d % 64 || I % 32) return MOE_ERR_UNSUPPORTED;
  } else if (D->act_dtype == MOE_BF16) {
    if (D->expert_dtype != MOE_BF16 && D->expert_dtype != MOE_MXFP8) return MOE_ERR_UNSUPPORTED;
    if (d % 256 || I % 128) return MOE_ERR_UNSUPPORTED;
  } else {
    return MOE_ERR_INVALID_ARG;
  }
  if (D->stage_rows != 0 && D->stage_rows != 64 && D->stage_rows != 128 && D->stage_rows != 256)
    return MOE_ERR_UNSUPPORTED;
  if (D->n_producer_cus < 0) return MOE_ERR_INVALID_ARG;
  // routing options
  if (D->n_group < 0 || D->topk_group < 0 || !(D->routed_scale >= 0.0f) || D->routed_scale > 3.0e38f)
    return MOE_ERR_INVALID_ARG;
  if (D->n_group > 1 && (D->n_group > 64 || E % D->n_group || D->topk_group < 1 || D->topk_group > D->n_group ||
                         k > D->topk_group * (E / D->n_group)))
    return MOE_ERR_INVALID_ARG;
  if (((D->flags & MOE_FLAG_BIAS_SELECT_ONLY) || D->n_group > 1) && D->score != MOE_SCORE_SIGMOID)
    return MOE_ERR_UNSUPPORTED;
  p->T = T; p->d = d; p->E = E; p->k = k; p->I = I; p->R = T * k;
  p->macro = macro;
  p->T_full = D->T;
  p->f32 = f32;
  p->mxfp8 = D->expert_dtype == MOE_MXFP8;
  p->act_es = f32 ? 4 : 2;
  p->nb = cdiv(T, kTokBlock);
  p->S = (!f32 && d % 1024 == 0 && d >= 2048) ? 4 : 1;
  if (f32) {
    p->BM = TileF32::BM;
    p->nN1 = I / 32;
    p->nN2 = d / 64;
  } else {
    // auto: 256-row stages (the 256 x 256 tile) once the bf16 experts
    // average 256 routed rows or more, else 128 (measured: 128 wins at
    // about 128 rows an expert, 256 from 256 rows up)
    const bool long_experts = !p->mxfp8 && (int64_t)T * k >= (int64_t)256 * E;
    p->BM = D->stage_rows ? D->stage_rows : (long_experts ? 256 : 128);
    // column tiles: the bf16 forward uses the 256-wide direct-to-LDS
    // tiles, MXFP8 128-wide tiles
    if (p->mxfp8 && p->BM != 128) return MOE_ERR_UNSUPPORTED;  // MXFP8 tiles have 128 rows
    static_assert(TileD256::BN == TileD256w::BN && TileD256h::BN == TileD256::BN, "one column width");
    const int bn = !p->mxfp8 ? TileD256::BN : TileB128::BN;
    p->nN1 = I / (bn / 2);
    p->nN2 = d / bn;
  }
  p->nC = cdiv(T, kCombTok);
  // row tiles of the forward (BM rows) and of the backward (TileDH::BM rows)
  const int min_bm = p->BM < TileDH::BM ? p->BM : TileDH::BM;
  p->max_tiles = p->R / min_bm + (E < p->R ? E : p->R) + 1;
  p->bwd_ok = !f32 && d % 128 == 0 && I % 128 == 0;
  p->nNdh = I / TileDH::BN;
  p->nNdx = d / TileDH::BN;
  p->nW2m = d / TileDW::BM;
  p->nW2n = I / TileDW::BN;
  p->nW13m = I / (TileDW::BM / 2);
  p->nW13n = d / TileDW::BN;
  p->nRP = cdiv(T, kPrepTok);

  const size_t R = (size_t)p->R, es = p->act_es;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = o; o = align256(o + bytes); return at; };
  p->n_ctr = C_HEADER + kMaxPhases * kXcds + p->nb + 3 * (size_t)p->max_tiles + 2 * (size_t)E + 16;
  p->o_ctr = take(p->n_ctr * 4);
  // router slices: each slice starts on a 128-byte line (a top-k task reads
  // the first rows of every slice while later slices' tasks may still run)
  p->lstride = slots::router_slice_stride(T, E);
  p->o_lpart = take((size_t)p->S * p->lstride * 4);
  p->o_topk = take(R * 4);
  p->o_gate = take(R * 4);
  p->o_bmask = take((size_t)p->nb * E * 8);
  p->o_bbase = take((size_t)p->nb * E * 4);
  p->o_counts = take((size_t)E * 4);
  p->o_offsets = take((size_t)(E + 1) * 4);
  p->o_tile_e = take((size_t)p->max_tiles * 4);
  p->o_tile_r0 = take((size_t)p->max_tiles * 4);
  p->o_tile_n = take((size_t)p->max_tiles * 4);
  p->o_perm = take(R * 4);
  p->o_inv = take(R * 4);
  p->o_src = take(R * 4);
  // the forward's source slots, one 128-byte multiple per row tile
  p->o_tsrc = take(slots::tile_slot(p->max_tiles, 0, p->BM, 1) * 4);
  p->o_grow = take(R * 4);
  p->o_etile = take((size_t)(E + 1) * 4);
  p->o_eoff = take((size_t)(E + 1) * 4);
  p->o_eorder = take((size_t)E * 4);
  p->o_h = take(R * I * es);
  // MXFP8 H scales by row-tile slot (BM rows of I/32 bytes: a multiple of
  // 128 bytes per tile, since I % 128 == 0)
  p->o_hs = take(slots::tile_slot(p->max_tiles, 0, p->BM, I / 32));
  p->o_xs = p->mxfp8 ? take((size_t)T * (d / 32)) : 0;
  p->o_big1 = take(R * d * es);
  p->o_big2 = take(R * d * es);
  p->mx_wgrad = p->mxfp8 && (D->flags & MOE_FLAG_MXFP8_WGRAD) != 0;
  if (p->bwd_ok && !fwd_only) {
    if (!p->mx_wgrad) p->o_gg = take(R * d * 2);
    p->o_zero = take(((size_t)2 * I + d + 256) * 2);
    p->o_dab = take(R * 2 * I * 2);
    p->o_dgp = take((size_t)p->nNdh * R * 4);
    if (p->mxfp8) {
      p->o_dyq = take((size_t)T * d);
      p->o_dys = take((size_t)T * (d / 32));
      p->o_dabq = take(R * 2 * I);
      p->o_dabs = take(R * 2 * (I / 32));
    }
    if (p->mx_wgrad) {
      // the weight gradients' operands along the rows, in row-tile slots
      p->kcap = p->max_tiles * TileDH::BM;
      const size_t kc = (size_t)p->kcap;
      p->o_xT = take((size_t)d * kc);
      p->o_xTs = take((size_t)d * (kc / 32));
      p->o_gT = take((size_t)d * kc);
      p->o_gTs = take((size_t)d * (kc / 32));
      p->o_hT = take((size_t)I * kc);
      p->o_hTs = take((size_t)I * (kc / 32));
      p->o_dabT = take((size_t)2 * I * kc);
      p->o_dabTs = take((size_t)2 * I * (kc / 32));
    }
  }
  if (!fwd_only) {
    p->o_rdz = take(R * 4);
    p->o_rpart = take((size_t)kRbSplits * E * d * 4);
    p->o_rpbias = take((size_t)kRbSplits * E * 4);
  }
  p->total = macro ? 2 * align256(o) : o;
  return MOE_OK;
}

template <class T>
static inline T* at(void* ws, size_t off) { return (T*)((char*)ws + off); }

static Sync make_sync(const Plan& p, void* ws, int32_t* status, uint32_t flags) {
  int* c = at<int>(ws, p.o_ctr);
  Sync s;
  s.queue = c + C_QUEUE;
  s.abort = c + C_ABORT;
  s.r2_done = c + C_R2;
  s.scan_done = c + C_SCAN;
  s.g2_done = c + C_G2;
  s.n_mtiles = c + C_NMT;
  s.aux3 = c + C_AUX3;
  s.q_done = c + C_QDONE;
  int* q = c + C_HEADER;
  s.qctr = q; q += kMaxPhases * kXcds;
  s.r1_cnt = q; q += p.nb;
  s.ready = q; q += p.max_tiles;
  s.h_cnt = q; q += p.max_tiles;
  s.aux0 = q; q += p.max_tiles;
  s.aux1 = q; q += p.E;
  s.aux2 = q; q += p.E;
  s.status = status;
  s.spin_limit = (flags & MOE_FLAG_SPIN_LIMIT_TINY) ? 64 : (1ll << 22);
  s.flags = flags;
  return s;
}

// The routing options of a descriptor (validated by make_plan).
static void set_routing(Fwd& F, const moe_desc* D) {
  F.select_only = (D->flags & MOE_FLAG_BIAS_SELECT_ONLY) ? 1 : 0;
  F.n_group = D->n_group > 1 ? D->n_group : 0;
  F.topk_group = D->n_group > 1 ? D->topk_group : 0;
  F.scale = D->routed_scale > 0.0f ? D->routed_scale : 1.0f;
}

static Fwd make_fwd(const Plan& p, const moe_desc* D, void* ws, const moe_saved* sv) {
  Fwd F;
  memset(&F, 0, sizeof(F));
  set_routing(F, D);
  F.T = p.T; F.d = p.d; F.E = p.E; F.k = p.k; F.I = p.I; F.R = p.R;
  F.nb = p.nb; F.S = p.S; F.BM = p.BM; F.nN1 = p.nN1; F.nN2 = p.nN2; F.nC = p.nC;
  F.max_tiles = p.max_tiles;
  F.score = D->score; F.renorm = D->renorm ? 1 : 0;
  // MXFP8 always pulls token rows from the quantised x (no gathered copy)
  F.direct = p.mxfp8 || ((D->flags & MOE_FLAG_DIRECT_PULL) && !p.f32) ? 1 : 0;
  F.lpart = at<float>(ws, p.o_lpart);
  F.lstride = p.lstride;
  F.logits = sv ? sv->logits : nullptr;
  F.topk = (sv && sv->topk_idx) ? sv->topk_idx : at<int>(ws, p.o_topk);
  F.gate = (sv && sv->gate) ? sv->gate : at<float>(ws, p.o_gate);
  F.bmask = at<unsigned long long>(ws, p.o_bmask);
  F.bbase = at<int>(ws, p.o_bbase);
  F.counts = (sv && sv->counts) ? sv->counts : at<int>(ws, p.o_counts);
  F.offsets = (sv && sv->offsets) ? sv->offsets : at<int>(ws, p.o_offsets);
  F.tile_e = at<int>(ws, p.o_tile_e);
  F.tile_r0 = at<int>(ws, p.o_tile_r0);
  F.tile_n = at<int>(ws, p.o_tile_n);
  F.etile = at<int>(ws, p.o_etile);
  F.perm = (sv && sv->perm) ? sv->perm : at<int>(ws, p.o_perm);
  F.inv = (sv && sv->inv) ? sv->inv : at<int>(ws, p.o_inv);
  F.tsrc = at<int>(ws, p.o_tsrc);
  F.grow = nullptr;
  F.xp = at<char>(ws, p.o_big1);
  F.a = sv ? sv->a : nullptr;
  F.b = sv ? sv->b : nullptr;
  F.h = (sv && sv->h) ? sv->h : at<char>(ws, p.o_h);
  F.yp = at<char>(ws, p.o_big2);
  if (p.mxfp8) {
    // H codes take the workspace H; H itself is written only if asked for
    F.h = sv ? sv->h : nullptr;
    F.hq = at<uint8_t>(ws, p.o_h);
    F.hs = at<uint8_t>(ws, p.o_hs);
    F.xq = at<uint8_t>(ws, p.o_big1);
    F.xs = at<uint8_t>(ws, p.o_xs);
  }
  F.s = make_sync(p, ws, sv ? sv->status : nullptr, D->flags);
  return F;
}

// ------------------------------------------------------------------ kernels
__global__ void k_zero(int* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// Workgroups per CU a tile's kernel is compiled for: two for the 128-row
// register-staged tiles, one for 256-row tiles and for the direct-to-LDS
// ring (its LDS holds one).
template <class TL>
constexpr int tile_occupancy() {
  return (TL::BM == 128 && !TL::kDMA) ? 2 : 1;
}

// Spreads consecutive logical tiles over one XCD: hardware dispatches
// workgroup b to XCD b % 8, so logical tile ranges stay in one L2.
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int per = n / 8, rem = n % 8, x = b % 8, s = b / 8;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + s;
}

template <class Act>
__global__ void __launch_bounds__(256) k_router_partial(Fwd F) { router_partial<Act>(F, blockIdx.x); }

template <bool MASKS>
__global__ void __launch_bounds__(256) k_router_topk(Fwd F) {
  extern __shared__ __align__(16) char smem[];
  router_topk<MASKS>(F, blockIdx.x, smem);
}

__global__ void __launch_bounds__(256) k_build_masks(Fwd F) {
  __shared__ unsigned long long smask[kMaxE];
  build_masks(F, blockIdx.x, smask);
}

__global__ void __launch_bounds__(256) k_scan(Fwd F) {
  __shared__ int sh[2 * kMaxE + 16];
  layout_scan<false>(F, sh);
}

template <class Act, bool COPY>
__global__ void __launch_bounds__(256) k_gather(Fwd F) {
  __shared__ int ssrc[256];
  const int tile = blockIdx.x;
  if (tile >= *F.s.n_mtiles) return;
  gather_tile<Act, COPY, false>(F, tile, ssrc);
}

// The bf16 tiles take their narrower variants for short row tiles: at most
// 64 rows the 64-row tile, at most 128 rows (of a 256-row stage) the
// 128-row one.
template <class TL>
constexpr bool has_half_tile() {
  return std::is_same<TL, TileD256>::value || std::is_same<TL, TileD256w>::value;
}
template <class TL>
constexpr size_t fwd_tile_lds() {
  if constexpr (std::is_same<TL, TileD256w>::value)
    return TileD256w::smem_bytes > TileD256::smem_bytes ? TileD256w::smem_bytes : TileD256::smem_bytes;
  else
    return TL::smem_bytes;
}

// CO: the tile's output has a reader in the same launch (stored coherently).
template <class Act, class TL, bool CO>
__device__ __forceinline__ void run_g1(const Fwd& F, int tile, int nt, char* smem) {
  if constexpr (std::is_same<Act, float>::value)
    g1_tile_f32<CO>(F, tile, nt, (float*)smem);
  else if constexpr (TL::kMX)
    g1_tile_mx<TL, CO>(F, tile, nt, (bf16_t*)smem);
  else if constexpr (has_half_tile<TL>()) {
    const int n = fwd_tile(F, tile).n;
    if (n <= TileD256h::BM)
      g1_tile_bf16<TileD256h, CO>(F, tile, nt, (bf16_t*)smem);
    else if (TL::BM > TileD256::BM && n <= TileD256::BM)
      g1_tile_bf16<TileD256, CO>(F, tile, nt, (bf16_t*)smem);
    else
      g1_tile_bf16<TL, CO>(F, tile, nt, (bf16_t*)smem);
  }
  else
    g1_tile_bf16<TL, CO>(F, tile, nt, (bf16_t*)smem);
}
template <class Act, class TL, bool CO>
__device__ __forceinline__ void run_g2(const Fwd& F, int tile, int nt, char* smem) {
  if constexpr (std::is_same<Act, float>::value)
    g2_tile_f32<CO>(F, tile, nt, (float*)smem);
  else if constexpr (TL::kMX)
    g2_tile_mx<TL, CO>(F, tile, nt, (bf16_t*)smem);
  else if constexpr (has_half_tile<TL>()) {
    const int n = fwd_tile(F, tile).n;
    if (n <= TileD256h::BM)
      g2_tile_bf16<TileD256h, CO>(F, tile, nt, (bf16_t*)smem);
    else if (TL::BM > TileD256::BM && n <= TileD256::BM)
      g2_tile_bf16<TileD256, CO>(F, tile, nt, (bf16_t*)smem);
    else
      g2_tile_bf16<TL, CO>(F, tile, nt, (bf16_t*)smem);
  }
  else
    g2_tile_bf16<TL, CO>(F, tile, nt, (bf16_t*)smem);
}

__global__ void __launch_bounds__(256) k_quant_tokens(Fwd F) { quant_tokens(F, blockIdx.x); }

template <class Act, class TL>
__global__ void __launch_bounds__(256, tile_occupancy<TL>()) k_g1(Fwd F) {
  extern __shared__ __align__(16) char smem[];
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  if (id >= *F.s.n_mtiles * F.nN1) return;
  int tile, nt;
  raster_decode(F.etile, F.E, F.nN1, id, tile, nt);
  run_g1<Act, TL, false>(F, tile, nt, smem);
}

template <class Act, class TL>
__global__ void __launch_bounds__(256, tile_occupancy<TL>()) k_g2(Fwd F) {
  extern __shared__ __align__(16) char smem[];
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  if (id >= *F.s.n_mtiles * F.nN2) return;
  int tile, nt;
  raster_decode(F.etile, F.E, F.nN2, id, tile, nt);
  run_g2<Act, TL, false>(F, tile, nt, smem);
}

// The combine as a plain launch after the persistent ones: nothing to merge
// once a bounded wait of the call has given up (the rows were not computed).
template <class Act>
__global__ void __launch_bounds__(256) k_combine(Fwd F) {
  if (load_relaxed(F.s.abort)) return;
  combine_tokens<Act>(merge_of(F), blockIdx.x);
}

// The same merge for moe_combine (no call state to consult).
template <class Act>
__global__ void __launch_bounds__(256) k_combine_alone(Fwd F) {
  combine_tokens<Act>(merge_of(F), blockIdx.x);
}

// The persistent forward: phases router slices (+ the MXFP8 quantisation
// of x by token block) | top-k | layout | gather | up-projection tiles |
// down-projection tiles | combine, claimed through
// the per-XCD phase queues (sched.h); the projection tiles are enumerated
// in the grouped raster, 64 consecutive tasks per XCD queue block.  Each
// task waits on the counters its inputs raise.
// A task's signal releases its stores at agent scope only when a phase
// that reads them runs in this launch (MASK); readers in later launches see
// them through the kernel boundary.
// Phases a workgroup claims under the CU partition: producers (workgroups
// below n_prod) routing, layout, gather and combine; consumers the GEMMs.
constexpr unsigned kProducerPhases = 0x4Fu, kConsumerPhases = 0x30u;

// Each workgroup copies the row-tile boundaries of the experts (etile, E+1
// ints) into LDS at its first GEMM task, for the raster decode's binary
// search (eight dependent global loads per task otherwise).
constexpr int kEtileLds = kMaxE + 1;

// RING: a launch of the macrobatch ring, whose first phase also runs the
// previous macrobatch's merge (instantiated apart: the merge's registers
// would otherwise weigh on every other launch's routing phase).
template <class Act, class TL, unsigned MASK, bool RING = false>
__global__ void __launch_bounds__(256, tile_occupancy<TL>()) k_fused_fwd(Fwd F) {
  extern __shared__ __align__(16) char smem[];
  __shared__ Claim c;
  __shared__ int s_flag;
  __shared__ int s_etile[kEtileLds];
  bool etile_lds = false;
  const unsigned roles = F.n_prod == 0 ? 0x7Fu : ((int)blockIdx.x < F.n_prod ? kProducerPhases : kConsumerPhases);
  if (threadIdx.x == 0) {
    c.phase = 0;
    c.qoff = 0;
    c.own = claim_home(F.s.flags);
    c.nmt = -1;
  }
  for (;;) {
    __syncthreads();
    if (threadIdx.x == 0) {
      const WaitCtx W = wctx(F.s);
      auto shape = [&](int ph, int& groups, int& per) -> bool {
        per = 1;
        groups = 0;
        if (!((MASK >> ph) & 1u)) return true;  // phase run by another launch
        if (!((roles >> ph) & 1u)) return true;  // phase of the other side of the partition
        if (ph == 0) { groups = F.nb * F.S + (TL::kMX ? F.nb : 0) + (RING ? F.prev_nC : 0); return true; }
        if (ph == 1) { groups = F.nb * kTopkChunks; return true; }
        if (ph == 2) { groups = 1; return true; }
        if (c.nmt < 0) {
          if (!thread_wait_geq(F.s.scan_done, 1, W)) return false;
          c.nmt = load_relaxed(F.s.n_mtiles);
        }
        if (ph == 3) { groups = c.nmt; return true; }
        if (ph == 6) { groups = F.nC; return true; }
        groups = cdiv(c.nmt * (ph == 4 ? F.nN1 : F.nN2), kRasterBlock);
        per = kRasterBlock;
        return true;
      };
      c.task = claim_next(F.s.qctr, 7, c, shape);
    }
    __syncthreads();
    const int t = c.task, ph = c.phase;
    if (t < 0) break;
    const WaitCtx W = wctx(F.s);
    const int s_nmt = c.nmt;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if ((ph == 4 || ph == 5) && !etile_lds) {
      // the layout is complete (the claim waited for it)
      for (int e = threadIdx.x; e <= F.E; e += kThreads) s_etile[e] = F.etile[e];
      __syncthreads();
      etile_lds = true;
    }
    // A task whose wait fails (timeout or abort) does no work and raises
    // no counter (protocol.h).
    if ((MASK & 1u) && ph == 0) {
      const int nr = F.nb * F.S + (TL::kMX ? F.nb : 0);
      if (RING && t >= nr) {
        // the previous macrobatch's merge (its operands are complete)
        if constexpr (RING)
          if (!load_relaxed(F.prev_abort)) combine_tokens<Act>(F.prev, t - nr);
      } else if (TL::kMX && t >= F.nb * F.S) {
        quant_tokens(F, t - F.nb * F.S);
        signal_add<(MASK & 0x18u) != 0>(F.s.q_done, 1);  // read by gather, g1
      } else {
        router_partial<Act, !TL::kMX>(F, t);
        if constexpr ((MASK & 2u) != 0)
          signal_add_stored(&F.s.r1_cnt[t / F.S], 1);
        else
          signal_add<false>(&F.s.r1_cnt[t / F.S], 1);
      }
    } else if ((MASK & 2u) && ph == 1) {
      if (!wait_geq(&F.s.r1_cnt[t / kTopkChunks], F.S, W, &s_flag)) continue;
      router_topk<true>(F, t, smem);
      // read by scan, gather, combine (stored coherently)
      if constexpr ((MASK & 0x4Cu) != 0)
        signal_add_stored(F.s.r2_done, 1);
      else
        signal_add<false>(F.s.r2_done, 1);
    } else if ((MASK & 4u) && ph == 2) {
      if (!wait_geq(F.s.r2_done, F.nb * kTopkChunks, W, &s_flag)) continue;
      layout_scan<(MASK & 0x78u) != 0>(F, (int*)smem);
      if constexpr ((MASK & 0x78u) != 0)
        signal_add_stored(F.s.scan_done, 1);  // the layout is stored coherently
      else
        signal_add<false>(F.s.scan_done, 1);
    } else if ((MASK & 8u) && ph == 3) {
      // MXFP8: a row tile is ready once the codes of x are complete too
      if (TL::kMX && !wait_geq(F.s.q_done, F.nb, W, &s_flag)) continue;
      if (F.direct)
        gather_tile<Act, false, (MASK & 0x50u) != 0>(F, t, (int*)smem);  // read by g1, combine
      else
        gather_tile<Act, true, (MASK & 0x50u) != 0>(F, t, (int*)smem);
    } else if ((MASK & 16u) && ph == 4) {
      if (t >= s_nmt * F.nN1) continue;
      int tile, nt;
      raster_decode(s_etile, F.E, F.nN1, t, tile, nt);
      if (!wait_geq(&F.s.ready[tile], 1, W, &s_flag)) continue;
      run_g1<Act, TL, (MASK & 32u) != 0>(F, tile, nt, smem);
      // H (or its codes) is stored coherently: with the down projection in
      // this launch the count waits for those stores, with no L2 write-back
      if constexpr ((MASK & 32u) != 0)
        signal_add_stored(&F.s.h_cnt[tile], 1);
      else
        signal_add<false>(&F.s.h_cnt[tile], 1);
    } else if ((MASK & 32u) && ph == 5) {
      if (t >= s_nmt * F.nN2) continue;
      int tile, nt;
      raster_decode(s_etile, F.E, F.nN2, t, tile, nt);
      if (!wait_geq(&F.s.h_cnt[tile], F.nN1, W, &s_flag)) continue;
      run_g2<Act, TL, (MASK & 64u) != 0>(F, tile, nt, smem);
      if constexpr ((MASK & 64u) != 0)
        signal_add_stored(F.s.g2_done, 1);  // rows stored coherently
      else
        signal_add<false>(F.s.g2_done, 1);
    } else if ((MASK & 64u) && ph == 6) {
      // inv comes from this launch's gather tasks when it runs them
      if (wait_geq(F.s.g2_done, s_nmt * F.nN2, W, &s_flag)) combine_tokens<Act, (MASK & 8u) != 0>(merge_of(F), t);
    }
  }
}

// Standalone pull gather: xp[r] = x[perm[r] / k].
template <class Act>
__global__ void __launch_bounds__(256) k_gather_perm(const Act* __restrict__ x, const int* __restrict__ perm,
                                                     Act* __restrict__ xp, int R, int d, int k) {
  const int nvec = d * (int)sizeof(Act) / 16;
  for (int r = blockIdx.x * 4 + (threadIdx.x >> 6); r < R; r += gridDim.x * 4) {
    const int a = perm[r];
    if ((unsigned)a >= (unsigned)R) continue;  // outside [0, R): the row is left unwritten
    wave_copy_row((const uint4*)x + (size_t)(a / k) * nvec, (uint4*)xp + (size_t)r * nvec, nvec, CopyAsIs());
  }
}

// Token-major gather: each wave reads one token row once and writes it to
// the k rows the layout gave that token, xp[inv[t k + j]] = x[t].  Same
// rows as the pull by perm, with x read once instead of k times.  A row
// index outside [0, R) is skipped.  k <= 64 (the plan caps k at 16).
template <class Act>
__global__ void __launch_bounds__(256) k_gather_push(const Act* __restrict__ x, const int* __restrict__ inv,
                                                     Act* __restrict__ xp, int T, int R, int d, int k) {
  const int nvec = d * (int)sizeof(Act) / 16;
  const int lane = threadIdx.x & 63;
  for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < T; t += gridDim.x * 4) {
    const int lane_row = lane < k ? inv[(size_t)t * k + lane] : -1;
    wave_push_row((const uint4*)x + (size_t)t * nvec, (uint4*)xp, nvec, k, R, lane_row,
                  [](int, uint4 u) { return u; });
  }
}

// ------------------------------------------------------------------ backward
__global__ void __launch_bounds__(256) k_bwd_setup(Bwd B) {
  __shared__ int sh[2 * kMaxE + 16];
  bwd_setup(B, sh);
}

__global__ void __launch_bounds__(256) k_bwd_rowprep(Bwd B) { bwd_rowprep(B, blockIdx.x); }

// Setup (block 0) and row preparation (blocks 1 ..) ahead of the persistent
// backward launches, as one plain launch: neither reads what the other
// writes, the launch boundary publishes both, and each block still raises
// the count that the later launches' claims wait on.  (At the DeepSeek-V3
// shape 186 us, against 196-210 us as a persistent launch; the row pulls
// write 0.94 GB.)
__global__ void __launch_bounds__(256) k_bwd_prep(Bwd B) {
  __shared__ int sh[2 * kMaxE + 16];
  if (blockIdx.x == 0)
    bwd_setup(B, sh);
  else
    bwd_rowprep(B, blockIdx.x - 1);
  signal_add<false>(B.s.scan_done, 1);
}

__global__ void __launch_bounds__(256, 2) k_bwd_dh(Bwd B) {
  extern __shared__ __align__(16) char smem[];
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  if (id >= *B.s.n_mtiles * B.nNdh) return;
  int tile, nt;
  raster_decode(B.etile, B.E, B.nNdh, id, tile, nt);
  bwd_dh_tile(B, tile, nt, (bf16_t*)smem, (float*)smem);
}

__global__ void __launch_bounds__(256, 2) k_bwd_dxp(Bwd B) {
  extern __shared__ __align__(16) char smem[];
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  if (id >= *B.s.n_mtiles * B.nNdx) return;
  int tile, nt;
  raster_decode(B.etile, B.E, B.nNdx, id, tile, nt);
  bwd_dxp_tile(B, tile, nt, (bf16_t*)smem);
}

__global__ void __launch_bounds__(256, 2) k_bwd_dh_mx(Bwd B) {
  extern __shared__ __align__(16) char smem[];
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  if (id >= *B.s.n_mtiles * B.nNdh) return;
  int tile, nt;
  raster_decode(B.etile, B.E, B.nNdh, id, tile, nt);
  bwd_dh_tile_mx(B, tile, nt, (bf16_t*)smem);
}

__global__ void __launch_bounds__(256, 2) k_bwd_dxp_mx(Bwd B) {
  extern __shared__ __align__(16) char smem[];
  const int id = xcd_remap(blockIdx.x, gridDim.x);
  if (id >= *B.s.n_mtiles * B.nNdx) return;
  int tile, nt;
  raster_decode(B.etile, B.E, B.nNdx, id, tile, nt);
  bwd_dxp_tile_mx(B, tile, nt, (bf16_t*)smem);
}

__global__ void __launch_bounds__(256, 2) k_bwd_dw2(Bwd B) {
  extern __shared__ __align__(16) char smem[];
  // dispatch order (heaviest experts first) spread round-robin over the XCDs
  const int per = B.nW2m * cdiv(B.nW2n, kWgradPerTicket);
  bwd_dw2_band(B, blockIdx.x / per, blockIdx.x % per, (bf16_t*)smem);
}

__global__ void __launch_bounds__(256, 2) k_bwd_dw13(Bwd B) {
  extern __shared__ __align__(16) char smem[];
  const int per = B.nW13m * cdiv(B.nW13n, kWgradPerTicket);
  bwd_dw13_band(B, blockIdx.x / per, blockIdx.x % per, (bf16_t*)smem);
}

__global__ void __launch_bounds__(256, 2) k_bwd_dw2_mx(Bwd B) {
  extern __shared__ __align__(16) char smem[];
  const int per = B.nW2m * cdiv(B.nW2n, kWgradPerTicket);
  bwd_dw2_band_mx(B, blockIdx.x / per, blockIdx.x % per, (bf16_t*)smem);
}

__global__ void __launch_bounds__(256, 2) k_bwd_dw13_mx(Bwd B) {
  extern __shared__ __align__(16) char smem[];
  const int per = B.nW13m * cdiv(B.nW13n, kWgradPerTicket);
  bwd_dw13_band_mx(B, blockIdx.x / per, blockIdx.x % per, (bf16_t*)smem);
}

// dX as a plain launch after the persistent ones (skipped when a bounded
// wait of the call gave up: the rows it sums were not computed).
__global__ void __launch_bounds__(256) k_bwd_dx(Bwd B) {
  if (load_relaxed(B.s.abort)) return;
  bwd_dx_tokens(B, blockIdx.x);
}

// The persistent backward: phases setup | rowprep | dh | dw2 | dxp | dw13
// | dx through the per-XCD phase queues (dh and dxp tiles in the grouped
// raster, 64 per queue block; the weight-gradient bands of each expert cut
// into 8 slices of consecutive bands, slice x on queue x, experts in order
// of decreasing load on every queue; one band of kWgradPerTicket column
// tiles per claim).
// Workgroups per CU the persistent backward asks the compiler to fit: two
// where the phases' registers allow it without spilling, else one.
constexpr int bwd_occupancy(unsigned mask) {
  return mask == 0x7Fu || mask == 0x57u || mask == 0x28u ? 1 : 2;
}

// MX: every GEMM task takes the MXFP8 tiles (bwd_mx.h).
template <unsigned MASK, bool MX = false>
__global__ void __launch_bounds__(256, bwd_occupancy(MASK)) k_fused_bwd(Bwd B) {
  extern __shared__ __align__(16) char smem[];
  __shared__ Claim c;
  __shared__ int s_flag;
  __shared__ int s_etile[(MASK & 0x14u) ? kEtileLds : 1];  // dh and dxp tiles only
  bool etile_lds = false;
  if (threadIdx.x == 0) {
    c.phase = 0;
    c.qoff = 0;
    c.own = claim_home(B.s.flags);
    c.nmt = -1;
  }
  for (;;) {
    __syncthreads();
    if (threadIdx.x == 0) {
      const WaitCtx W = wctx(B.s);
      const int g2 = B.nW2m * cdiv(B.nW2n, kWgradPerTicket), g13 = B.nW13m * cdiv(B.nW13n, kWgradPerTicket);
      auto shape = [&](int ph, int& groups, int& per) -> bool {
        per = 1;
        groups = 0;
        if (!((MASK >> ph) & 1u)) return true;  // phase run by another launch
        if (ph == 0) { groups = 1; return true; }
        if (ph == 1) { groups = B.nRP; return true; }
        if (ph == 3) { groups = 8 * B.E; per = cdiv(g2, 8); return true; }
        if (ph == 5) { groups = 8 * B.E; per = cdiv(g13, 8); return true; }
        if (c.nmt < 0) {
          if (!thread_wait_geq(B.s.scan_done, 1 + B.nRP, W)) return false;
          c.nmt = load_relaxed(B.s.n_mtiles);
        }
        if (ph == 6) { groups = B.nC; return true; }
        groups = cdiv(c.nmt * (ph == 2 ? B.nNdh : B.nNdx), kRasterBlock);
        per = kRasterBlock;
        return true;
      };
      c.task = claim_next(B.s.qctr, 7, c, shape);
    }
    __syncthreads();
    const int t = c.task, ph = c.phase;
    if (t < 0) break;
    const WaitCtx W = wctx(B.s);
    const int s_nmt = c.nmt;
    if constexpr ((MASK & 0x14u) != 0) {
      if ((ph == 2 || ph == 4) && !etile_lds) {
        // the row tiles are listed (the claim waited for setup)
        for (int e = threadIdx.x; e <= B.E; e += kThreads) s_etile[e] = B.etile[e];
        __syncthreads();
        etile_lds = true;
      }
    }
    const int g2 = B.nW2m * cdiv(B.nW2n, kWgradPerTicket), g13 = B.nW13m * cdiv(B.nW13n, kWgradPerTicket);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if ((MASK & 1u) && ph == 0) {
      bwd_setup(B, (int*)smem);
      signal_add<(MASK & 0x7Cu) != 0>(B.s.scan_done, 1);
    } else if ((MASK & 2u) && ph == 1) {
      bwd_rowprep(B, t);
      signal_add<(MASK & 0x7Cu) != 0>(B.s.scan_done, 1);
    } else if ((MASK & 0x28u) && (ph == 3 || ph == 5)) {
      // the expert order comes from setup
      if (!wait_geq(B.s.scan_done, 1 + B.nRP, W, &s_flag)) continue;
      const int per = ph == 3 ? g2 : g13, span = 8 * cdiv(per, 8);
      const int rank = t / span, band = t % span;
      if (band >= per) continue;  // the last slice's padding
      if ((MASK & 8u) && ph == 3) {
        if constexpr (MX)
          bwd_dw2_band_mx(B, rank, band, (bf16_t*)smem);
        else
          bwd_dw2_band(B, rank, band, (bf16_t*)smem);
      } else if (MASK & 0x20u) {
        const int e = min(max(B.eorder[min(rank, B.E - 1)], 0), B.E - 1);
        const int need = (B.etile[e + 1] - B.etile[e]) * B.nNdh;
        if (wait_geq(&B.s.aux1[e], need, W, &s_flag)) {
          if constexpr (MX)
            bwd_dw13_band_mx(B, rank, band, (bf16_t*)smem);
          else
            bwd_dw13_band(B, rank, band, (bf16_t*)smem);
        }
      }
    } else if ((MASK & 4u) && ph == 2) {
      if (t >= s_nmt * B.nNdh) continue;
      int tile, nt;
      raster_decode(s_etile, B.E, B.nNdh, t, tile, nt);
      // [dA | dB] is read by dxp and dw13, the dgate partials by dx: with dx
      // in this launch both are published by an agent-scope release; with
      // only dxp or dw13, [dA | dB] is stored coherently and the count waits
      // for those stores; otherwise the launch boundary publishes them
      constexpr bool CO = (MASK & 0x30u) != 0 && (MASK & 0x40u) == 0;
      if constexpr (MX)
        bwd_dh_tile_mx(B, tile, nt, (bf16_t*)smem);
      else
        bwd_dh_tile<CO>(B, tile, nt, (bf16_t*)smem, (float*)smem);
      if constexpr (CO && !MX)
        signal_add_stored(&B.s.h_cnt[tile], 1);
      else
        signal_add<(MASK & 0x70u) != 0>(&B.s.h_cnt[tile], 1);
      // the second count has nothing new to publish
      signal_add<false>(&B.s.aux1[bwd_tile(B, tile).e], 1);
    } else if ((MASK & 16u) && ph == 4) {
      if (t >= s_nmt * B.nNdx) continue;
      int tile, nt;
      raster_decode(s_etile, B.E, B.nNdx, t, tile, nt);
      if (!wait_geq(&B.s.h_cnt[tile], B.nNdh, W, &s_flag)) continue;
      if constexpr (MX)
        bwd_dxp_tile_mx(B, tile, nt, (bf16_t*)smem);
      else
        bwd_dxp_tile(B, tile, nt, (bf16_t*)smem);
      signal_add<(MASK & 64u) != 0>(B.s.g2_done, 1);
    } else if ((MASK & 64u) && ph == 6) {
      if (wait_geq(B.s.g2_done, s_nmt * B.nNdx, W, &s_flag)) bwd_dx_tokens(B, t);
    }
  }
}

// ------------------------------------------------------------------ host
// Compute units of the current device, asked on every call (the library
// keeps no state between calls, and the caller may switch devices).
static int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

template <class K>
static bool set_smem(K kernel, size_t bytes) {
  if (bytes <= 65536) return true;
  return hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) ==
         hipSuccess;
}

// Workgroups of a persistent kernel: as many as can be resident at once
// (more would only queue behind the first wave of workgroups).
template <class K>
static int persistent_grid(K kernel, size_t smem, int requested) {
  if (requested > 0) return requested;
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, smem) != hipSuccess || per_cu < 1)
    per_cu = 1;
  return per_cu * num_cus();
}

static int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// An automatic persistent grid larger than the most tasks any phase of the
// launch can have only adds workgroups that walk every phase's queues
// for nothing (at T = 64 the forward took 0.20 ms with 512 workgroups
// against 0.08 ms as separate kernels): the grid is capped there, at no
// fewer than one workgroup per XCD.  An explicit grid or a producer
// partition keeps its own size.
static int capped_grid(const moe_desc* D, int n_wg, long long most_tasks) {
  if (D->n_workgroups > 0 || D->n_producer_cus > 0) return n_wg;
  const long long cap = most_tasks > kXcds ? most_tasks : kXcds;
  return cap < n_wg ? (int)cap : n_wg;
}

// The most tasks of any phase in MASK of the forward (tile counts at their
// upper bound, max_tiles row tiles).
template <bool MX, bool RING>
static long long fwd_most_tasks(const Fwd& F, unsigned mask) {
  long long m = 1;
  auto up = [&](unsigned ph, long long n) { if ((mask >> ph) & 1u) m = n > m ? n : m; };
  up(0, (long long)F.nb * F.S + (MX ? F.nb : 0) + (RING ? F.prev_nC : 0));
  up(1, (long long)F.nb * kTopkChunks);
  up(3, F.max_tiles);
  up(4, (long long)F.max_tiles * F.nN1);
  up(5, (long long)F.max_tiles * F.nN2);
  up(6, F.nC);
  return m;
}

template <class Act, class TL, unsigned MASK, bool RING = false>
static int launch_fused_fwd(const moe_desc* D, const Fwd& F0, size_t smem, hipStream_t st) {
  if (!set_smem(k_fused_fwd<Act, TL, MASK, RING>, smem)) return MOE_ERR_HIP;
  const int resident = persistent_grid(k_fused_fwd<Act, TL, MASK, RING>, smem, 0);
  const int n_wg = capped_grid(D, persistent_grid(k_fused_fwd<Act, TL, MASK, RING>, smem, D->n_workgroups),
                               fwd_most_tasks<TL::kMX, RING>(F0, MASK));
  if (n_wg <= 0 || resident <= 0) return MOE_ERR_HIP;
  Fwd F = F0;
  F.n_prod = 0;
  if (D->n_producer_cus > 0 && (MASK & kProducerPhases) && (MASK & kConsumerPhases)) {
    // a consumer may wait on a producer task not yet claimed, so both sides
    // must be resident at once: the grid may not exceed the resident limit
    if (n_wg > resident) return MOE_ERR_INVALID_ARG;
    const int per_cu = resident / num_cus() > 0 ? resident / num_cus() : 1;
    F.n_prod = D->n_producer_cus * per_cu;
    if (F.n_prod >= n_wg) return MOE_ERR_INVALID_ARG;  // no consumer left
  }
  hipLaunchKernelGGL((k_fused_fwd<Act, TL, MASK, RING>), dim3(n_wg), dim3(256), smem, st, F);
  return launch_status();
}

// The same for the backward's phases.
static long long bwd_most_tasks(const Bwd& B, unsigned mask) {
  long long m = 1;
  auto up = [&](unsigned ph, long long n) { if ((mask >> ph) & 1u) m = n > m ? n : m; };
  up(1, B.nRP);
  up(2, (long long)B.max_tiles * B.nNdh);
  up(3, (long long)B.E * B.nW2m * cdiv(B.nW2n, kWgradPerTicket));
  up(4, (long long)B.max_tiles * B.nNdx);
  up(5, (long long)B.E * B.nW13m * cdiv(B.nW13n, kWgradPerTicket));
  up(6, B.nC);
  return m;
}

template <unsigned MASK, bool MX = false>
static int launch_fused_bwd(const moe_desc* D, const Bwd& B, size_t smem, hipStream_t st) {
  if (!set_smem(k_fused_bwd<MASK, MX>, smem)) return MOE_ERR_HIP;
  const int n_wg = capped_grid(D, persistent_grid(k_fused_bwd<MASK, MX>, smem, D->n_workgroups),
                               bwd_most_tasks(B, MASK));
  if (n_wg <= 0) return MOE_ERR_HIP;
  hipLaunchKernelGGL((k_fused_bwd<MASK, MX>), dim3(n_wg), dim3(256), smem, st, B);
  return launch_status();
}

// ring: a macrobatch of the ring (forward_in_batches): the default launch
// structure, and this macrobatch's merge is left to the next launch.
template <class Act, class TL>
static int forward_impl(const Plan& p, const moe_desc* D, const Fwd& F, hipStream_t st, bool ring = false) {
  constexpr bool isf = std::is_same<Act, float>::value;
  // the persistent kernel's LDS serves every task: GEMM stages, routing
  // masks (kMaxE u64), the layout scan (2 kMaxE + 16 ints), gather rows
  size_t smem = isf ? TileF32::smem_bytes : fwd_tile_lds<TL>();
  const size_t other[3] = {kTopkSmem, (2 * kMaxE + 16) * 4, 256 * 4};
  for (size_t o : other) smem = smem > o ? smem : o;
  const size_t gsmem = isf ? TileF32::smem_bytes : fwd_tile_lds<TL>();
  hipLaunchKernelGGL(k_zero, dim3(cdiv((int)p.n_ctr, 256)), dim3(256), 0, st, F.s.queue, (int)p.n_ctr);
  if (p.T == 0) {
    hipLaunchKernelGGL(k_scan, dim3(1), dim3(256), 0, st, F);
    return launch_status();
  }
  if (D->fused) {
    if (ring) {
      int rc = TL::kMX ? launch_fused_fwd<Act, TL, 0x1Fu, true>(D, F, smem, st)
                       : launch_fused_fwd<Act, TL, 0x3Fu, true>(D, F, smem, st);
      if (rc == MOE_OK && TL::kMX) rc = launch_fused_fwd<Act, TL, 0x20u>(D, F, smem, st);
      return rc;
    }
    if (D->flags & MOE_FLAG_PERSISTENT_SINGLE) return launch_fused_fwd<Act, TL, 0x7Fu>(D, F, smem, st);
    if (D->flags & MOE_FLAG_PERSISTENT_SPLIT) {
      // the same persistent scheduler, one launch per phase group
      int rc = launch_fused_fwd<Act, TL, 0x0Fu>(D, F, smem, st);
      if (rc == MOE_OK) rc = launch_fused_fwd<Act, TL, 0x10u>(D, F, smem, st);
      if (rc == MOE_OK) rc = launch_fused_fwd<Act, TL, 0x20u>(D, F, smem, st);
      if (rc == MOE_OK) rc = launch_fused_fwd<Act, TL, 0x40u>(D, F, 0, st);
      return rc;
    }
    // MXFP8: H's scale bytes are 2-byte pieces per row and column tile, and
    // storing them coherently for a reader in the same launch costs more
    // than the launch boundary (measured at the DeepSeek-V3 shape, T = 8192:
    // 6.16 ms in one launch against 5.99 ms), so the down projection gets a
    // launch of its own; so does the up projection, whose launch then
    // carries no routing, quantisation or gather code and spills no
    // registers (40-48 VGPRs with them): 6.02-6.03 against 6.11-6.14 ms
    if ((D->flags & MOE_FLAG_PERSISTENT_GEMM_APART) || TL::kMX) {
      // routing through the up projection (MXFP8: routing through the
      // gather | the up projection) | the down projection | combine
      int rc = TL::kMX ? launch_fused_fwd<Act, TL, 0x0Fu>(D, F, smem, st)
                       : launch_fused_fwd<Act, TL, 0x1Fu>(D, F, smem, st);
      if (rc == MOE_OK && TL::kMX) rc = launch_fused_fwd<Act, TL, 0x10u>(D, F, smem, st);
      if (rc == MOE_OK) rc = launch_fused_fwd<Act, TL, 0x20u>(D, F, smem, st);
      if (rc != MOE_OK) return rc;
      hipLaunchKernelGGL(k_combine<Act>, dim3(p.nC), dim3(256), 0, st, F);
      return launch_status();
    }
    // Routing through the down projection in one persistent launch: an
    // up-projection tile starts once its rows are staged, a down-projection
    // tile once every up-projection tile of its rows has stored H (stored
    // coherently, so publishing it writes no L2 back).  The combine then
    // runs as a plain launch, one workgroup per task: the launch boundary
    // orders it after every down-projection tile, and as a persistent phase
    // it only adds the claiming (measured: 149 us persistent against 105 us
    // plain at the DeepSeek-V3 shape).
    int rc = launch_fused_fwd<Act, TL, 0x3Fu>(D, F, smem, st);
    if (rc != MOE_OK) return rc;
    hipLaunchKernelGGL(k_combine<Act>, dim3(p.nC), dim3(256), 0, st, F);
    return launch_status();
  }
  hipLaunchKernelGGL(k_router_partial<Act>, dim3(p.nb * p.S), dim3(256), 0, st, F);
  if (!set_smem(k_router_topk<true>, kTopkSmem)) return MOE_ERR_HIP;
  hipLaunchKernelGGL(k_router_topk<true>, dim3(p.nb * kTopkChunks), dim3(256), kTopkSmem, st, F);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(256), 0, st, F);
  if (TL::kMX) hipLaunchKernelGGL(k_quant_tokens, dim3(p.nb), dim3(256), 0, st, F);
  if (F.direct)
    hipLaunchKernelGGL((k_gather<Act, false>), dim3(p.max_tiles), dim3(256), 0, st, F);
  else
    hipLaunchKernelGGL((k_gather<Act, true>), dim3(p.max_tiles), dim3(256), 0, st, F);
  if (!set_smem(k_g1<Act, TL>, gsmem) || !set_smem(k_g2<Act, TL>, gsmem)) return MOE_ERR_HIP;
  hipLaunchKernelGGL((k_g1<Act, TL>), dim3(p.max_tiles * p.nN1), dim3(256), gsmem, st, F);
  hipLaunchKernelGGL((k_g2<Act, TL>), dim3(p.max_tiles * p.nN2), dim3(256), gsmem, st, F);
  hipLaunchKernelGGL(k_combine<Act>, dim3(p.nC), dim3(256), 0, st, F);
  return launch_status();
}

static int backward_impl(const Plan& p, const moe_desc* D, const void* dy, const void* x, const moe_weights* w,
                         const moe_saved* sv, void* dx, void* dw1, void* dw3, void* dw2, float* dgate, void* ws,
                         hipStream_t st) {
  Bwd B;
  memset(&B, 0, sizeof(B));
  B.T = p.T; B.d = p.d; B.E = p.E; B.k = p.k; B.I = p.I; B.R = p.R; B.BM = TileDH::BM;
  B.max_tiles = p.max_tiles;
  B.nNdh = p.nNdh; B.nNdx = p.nNdx; B.nW2m = p.nW2m; B.nW2n = p.nW2n; B.nW13m = p.nW13m; B.nW13n = p.nW13n;
  B.nRP = p.nRP; B.nC = p.nC;
  B.dy = (const bf16_t*)dy; B.x = (const bf16_t*)x;
  B.w1 = (const bf16_t*)w->w1; B.w3 = (const bf16_t*)w->w3; B.w2 = (const bf16_t*)w->w2;
  B.gate = sv->gate; B.offsets = sv->offsets; B.perm = sv->perm; B.inv = sv->inv;
  B.a = (const bf16_t*)sv->a; B.b = (const bf16_t*)sv->b; B.h = (const bf16_t*)sv->h;
  B.dx = (bf16_t*)dx; B.dw1 = (bf16_t*)dw1; B.dw3 = (bf16_t*)dw3; B.dw2 = (bf16_t*)dw2; B.dgate = dgate;
  B.tile_e = at<int>(ws, p.o_tile_e); B.tile_r0 = at<int>(ws, p.o_tile_r0); B.tile_n = at<int>(ws, p.o_tile_n);
  B.etile = at<int>(ws, p.o_etile); B.eorder = at<int>(ws, p.o_eorder); B.eoff = at<int>(ws, p.o_eoff);
  B.src = at<int>(ws, p.o_src); B.grow = at<float>(ws, p.o_grow);
  B.dab = at<bf16_t>(ws, p.o_dab); B.dxp = at<bf16_t>(ws, p.o_big2); B.dgp = at<float>(ws, p.o_dgp);
  B.zrow = at<bf16_t>(ws, p.o_zero);
  B.xp = at<bf16_t>(ws, p.o_big1);
  B.gg = at<bf16_t>(ws, p.o_gg);
  B.s = make_sync(p, ws, sv->status, D->flags);
  hipLaunchKernelGGL(k_zero, dim3(cdiv((int)p.n_ctr, 256)), dim3(256), 0, st, B.s.queue, (int)p.n_ctr);
  const int nz = (int)(((size_t)2 * p.I + p.d + 256) / 2);
  hipLaunchKernelGGL(k_zero, dim3(cdiv(nz, 256)), dim3(256), 0, st, at<int>(ws, p.o_zero), nz);
  // weight-gradient tiles: their main loop's LDS plus the store staging
  const size_t sm_dh = TileDH::smem_bytes, sm_dw = TileDW::smem_bytes + kWgradStageBytes;
  if (p.mxfp8) {
    // MXFP8: the phases of the bf16 backward (persistent launches, one per
    // phase, or ordinary grids) on the MXFP8 tiles, with the quantisations
    // as plain launches in between: dY along d before dh; the weight
    // gradients' x, g dY and H operands along the rows once the row tiles
    // and sources are known; [dA | dB] along I and along the rows after dh
    B.w1t = (const uint8_t*)w->w1; B.w3t = (const uint8_t*)w->w3; B.w2t = (const uint8_t*)w->w2;
    B.w1ts = w->w1_scale; B.w3ts = w->w3_scale; B.w2ts = w->w2_scale;
    B.dyq = at<uint8_t>(ws, p.o_dyq); B.dys = at<uint8_t>(ws, p.o_dys);
    B.dabq = at<uint8_t>(ws, p.o_dabq); B.dabs = at<uint8_t>(ws, p.o_dabs);
    auto al16 = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
    B.mx_wide_d = p.d % 512 == 0 && al16(B.dys) && al16(B.w2ts);
    B.mx_wide_i = p.I % 512 == 0 && al16(B.dabs) && al16(B.w1ts) && al16(B.w3ts);
    const bool mxw = p.mx_wgrad;
    B.mx = mxw ? 1 : 0;
    B.kcap = p.kcap;
    B.xT = at<uint8_t>(ws, p.o_xT); B.xTs = at<uint8_t>(ws, p.o_xTs);
    B.gT = at<uint8_t>(ws, p.o_gT); B.gTs = at<uint8_t>(ws, p.o_gTs);
    B.hT = at<uint8_t>(ws, p.o_hT); B.hTs = at<uint8_t>(ws, p.o_hTs);
    B.dabT = at<uint8_t>(ws, p.o_dabT); B.dabTs = at<uint8_t>(ws, p.o_dabTs);
    const size_t sm_mx = TileMX128::smem_bytes, sm_dwmx = TileMX128::smem_bytes + kWgradStageBytes;
    static_assert(2 * (TileMX128::smem_bytes + 1024 + 4 * kEtileLds) <= 160 * 1024, "two MXFP8 workgroups per CU");
    static_assert(2 * (TileMX128::smem_bytes + kWgradStageBytes + 1024) <= 160 * 1024,
                  "two MXFP8 weight-gradient workgroups per CU");
    // operand quantisation along the rows: x, g dY, H in one launch, [dA |
    // dB] after dh (every block of a listed row tile; the others exit)
    const dim3 gq3(cdiv(p.d > p.I ? p.d : p.I, kThreads), 4 * p.max_tiles, 3), gq1(cdiv(2 * p.I, kThreads), 4 * p.max_tiles, 1);
    if (D->fused) {
      int rc = p.R > 0 ? mxfp8_quantize_rows(B.dy, p.T, p.d, B.dyq, B.dys, st) : MOE_OK;
      hipLaunchKernelGGL(k_bwd_prep, dim3(1 + p.nRP), dim3(256), 0, st, B);
      if (mxw && p.R > 0) hipLaunchKernelGGL(k_mx_quant_tiles<0>, gq3, dim3(kThreads), 0, st, B);
      if (rc == MOE_OK) rc = launch_fused_bwd<0x04u, true>(D, B, sm_mx, st);
      if (rc == MOE_OK && p.R > 0) {
        rc = mxfp8_quantize_rows(B.dab, p.R, 2 * (int64_t)p.I, B.dabq, B.dabs, st);
        if (mxw) hipLaunchKernelGGL(k_mx_quant_tiles<3>, gq1, dim3(kThreads), 0, st, B);
      }
      if (rc == MOE_OK) rc = mxw ? launch_fused_bwd<0x08u, true>(D, B, sm_dwmx, st) : launch_fused_bwd<0x08u>(D, B, sm_dw, st);
      if (rc == MOE_OK) rc = launch_fused_bwd<0x10u, true>(D, B, sm_mx, st);
      if (rc == MOE_OK) rc = mxw ? launch_fused_bwd<0x20u, true>(D, B, sm_dwmx, st) : launch_fused_bwd<0x20u>(D, B, sm_dw, st);
      if (rc != MOE_OK) return rc;
      if (p.nC > 0) hipLaunchKernelGGL(k_bwd_dx, dim3(p.nC), dim3(256), 0, st, B);
      return launch_status();
    }
    if (!set_smem(k_bwd_dh_mx, sm_mx) || !set_smem(k_bwd_dxp_mx, sm_mx) || !set_smem(k_bwd_dw2_mx, sm_dwmx) ||
        !set_smem(k_bwd_dw13_mx, sm_dwmx) || !set_smem(k_bwd_dw2, sm_dw) || !set_smem(k_bwd_dw13, sm_dw))
      return MOE_ERR_HIP;
    hipLaunchKernelGGL(k_bwd_setup, dim3(1), dim3(256), 0, st, B);
    if (p.nRP > 0) hipLaunchKernelGGL(k_bwd_rowprep, dim3(p.nRP), dim3(256), 0, st, B);
    if (p.R > 0) {
      int rc = mxfp8_quantize_rows(B.dy, p.T, p.d, B.dyq, B.dys, st);
      if (rc != MOE_OK) return rc;
      if (mxw) hipLaunchKernelGGL(k_mx_quant_tiles<0>, gq3, dim3(kThreads), 0, st, B);
      hipLaunchKernelGGL(k_bwd_dh_mx, dim3(p.max_tiles * p.nNdh), dim3(256), sm_mx, st, B);
    }
    const dim3 g2(p.E * p.nW2m * cdiv(p.nW2n, kWgradPerTicket)), g13(p.E * p.nW13m * cdiv(p.nW13n, kWgradPerTicket));
    if (mxw)
      hipLaunchKernelGGL(k_bwd_dw2_mx, g2, dim3(256), sm_dwmx, st, B);
    else
      hipLaunchKernelGGL(k_bwd_dw2, g2, dim3(256), sm_dw, st, B);
    if (p.R > 0) {
      int rc = mxfp8_quantize_rows(B.dab, p.R, 2 * (int64_t)p.I, B.dabq, B.dabs, st);
      if (rc != MOE_OK) return rc;
      if (mxw) hipLaunchKernelGGL(k_mx_quant_tiles<3>, gq1, dim3(kThreads), 0, st, B);
      hipLaunchKernelGGL(k_bwd_dxp_mx, dim3(p.max_tiles * p.nNdx), dim3(256), sm_mx, st, B);
    }
    if (mxw)
      hipLaunchKernelGGL(k_bwd_dw13_mx, g13, dim3(256), sm_dwmx, st, B);
    else
      hipLaunchKernelGGL(k_bwd_dw13, g13, dim3(256), sm_dw, st, B);
    if (p.nC > 0) hipLaunchKernelGGL(k_bwd_dx, dim3(p.nC), dim3(256), 0, st, B);
    return launch_status();
  }
  if (D->fused) {
    const size_t smem = sm_dw > sm_dh ? sm_dw : sm_dh;
    static_assert(2 * (TileDW::smem_bytes + kWgradStageBytes + 1024) <= 160 * 1024,
                  "two weight-gradient workgroups per CU, with their static LDS");
    // By default each GEMM phase gets a persistent launch of its own: no
    // phase reads what another phase of its launch writes, each launch's
    // registers are those of its own task kinds, and [dA | dB] needs no
    // coherent stores.  dH and dXp in one launch (dXp tiles waiting on the
    // dH tiles of their rows) measured 7.05 against 6.99 ms as two at the
    // DeepSeek-V3 Zipf shape: the pair spills more registers than either
    // alone.  Every backward task in one launch does not fit two
    // workgroups' registers per CU (MOE_FLAG_PERSISTENT_SINGLE runs it
    // anyway).
    if (!(D->flags & (MOE_FLAG_PERSISTENT_SINGLE | MOE_FLAG_PERSISTENT_WGRAD_APART))) {
      // each persistent launch reserves the LDS its own tiles use; setup
      // with the row preparation before them, and the dX gather-sum after
      // them (ordered by the launch boundary, as the forward's combine), run
      // as plain launches
      hipLaunchKernelGGL(k_bwd_prep, dim3(1 + p.nRP), dim3(256), 0, st, B);
      int rc = launch_fused_bwd<0x04u>(D, B, sm_dh, st);
      if (rc == MOE_OK) rc = launch_fused_bwd<0x10u>(D, B, sm_dh, st);
      if (rc == MOE_OK) rc = launch_fused_bwd<0x08u>(D, B, sm_dw, st);
      if (rc == MOE_OK) rc = launch_fused_bwd<0x20u>(D, B, sm_dw, st);
      if (rc != MOE_OK) return rc;
      if (p.nC > 0) hipLaunchKernelGGL(k_bwd_dx, dim3(p.nC), dim3(256), 0, st, B);
      return launch_status();
    }
    if (D->flags & MOE_FLAG_PERSISTENT_WGRAD_APART) {
      int rc = launch_fused_bwd<0x57u>(D, B, smem, st);
      if (rc == MOE_OK) rc = launch_fused_bwd<0x28u>(D, B, smem, st);
      return rc;
    }
    return launch_fused_bwd<0x7Fu>(D, B, smem, st);
  }
  if (!set_smem(k_bwd_dh, sm_dh) || !set_smem(k_bwd_dxp, sm_dh) || !set_smem(k_bwd_dw2, sm_dw) ||
      !set_smem(k_bwd_dw13, sm_dw))
    return MOE_ERR_HIP;
  hipLaunchKernelGGL(k_bwd_setup, dim3(1), dim3(256), 0, st, B);
  if (p.nRP > 0) hipLaunchKernelGGL(k_bwd_rowprep, dim3(p.nRP), dim3(256), 0, st, B);
  if (p.R > 0) hipLaunchKernelGGL(k_bwd_dh, dim3(p.max_tiles * p.nNdh), dim3(256), sm_dh, st, B);
  hipLaunchKernelGGL(k_bwd_dw2, dim3(p.E * p.nW2m * cdiv(p.nW2n, kWgradPerTicket)), dim3(256), sm_dw, st, B);
  if (p.R > 0) hipLaunchKernelGGL(k_bwd_dxp, dim3(p.max_tiles * p.nNdx), dim3(256), sm_dh, st, B);
  hipLaunchKernelGGL(k_bwd_dw13, dim3(p.E * p.nW13m * cdiv(p.nW13n, kWgradPerTicket)), dim3(256), sm_dw, st,
                     B);
  if (p.nC > 0) hipLaunchKernelGGL(k_bwd_dx, dim3(p.nC), dim3(256), 0, st, B);
  return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_workspace_size(const moe_desc* desc, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  Plan p;
  int rc = make_plan(desc, &p);
  if (rc != MOE_OK) return rc;
  *bytes = p.total;
  return MOE_OK;
}

int moe_route(const moe_desc* desc, const float* logits, const float* bias, int32_t* topk_idx, float* gate,
              void* stream) {
  Plan p;
  int rc = make_plan(desc, &p);
  if (rc != MOE_OK) return rc;
  if (p.macro) return MOE_ERR_UNSUPPORTED;
  if (p.T > 0 && (!logits || !topk_idx || !gate)) return MOE_ERR_INVALID_ARG;
  if (p.T == 0) return MOE_OK;
  Fwd F;
  memset(&F, 0, sizeof(F));
  F.T = p.T; F.E = p.E; F.k = p.k; F.S = 1;
  F.score = desc->score; F.renorm = desc->renorm ? 1 : 0;
  set_routing(F, desc);
  F.lpart = (float*)logits;
  F.bias = bias;
  F.topk = topk_idx;
  F.gate = gate;
  if (!set_smem(k_router_topk<false>, kTopkSmem)) return MOE_ERR_HIP;
  hipLaunchKernelGGL(k_router_topk<false>, dim3(p.nb * kTopkChunks), dim3(256), kTopkSmem, (hipStream_t)stream,
                     F);
  return launch_status();
}

int moe_layout(const moe_desc* desc, const int32_t* topk_idx, int32_t* counts, int32_t* offsets, int32_t* perm,
               int32_t* inv, int32_t* status, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  int rc = make_plan(desc, &p);
  if (rc != MOE_OK) return rc;
  if (p.macro) return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets || (p.R > 0 && (!topk_idx || !perm || !inv))) return MOE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < p.total) return MOE_ERR_WORKSPACE;
  moe_saved sv;
  memset(&sv, 0, sizeof(sv));
  sv.topk_idx = (int32_t*)topk_idx;
  sv.counts = counts;
  sv.offsets = offsets;
  sv.perm = perm;
  sv.inv = inv;
  sv.status = status;
  Fwd F = make_fwd(p, desc, workspace, &sv);
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(k_zero, dim3(cdiv((int)p.n_ctr, 256)), dim3(256), 0, st, F.s.queue, (int)p.n_ctr);
  if (p.nb > 0) hipLaunchKernelGGL(k_build_masks, dim3(p.nb), dim3(256), 0, st, F);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(256), 0, st, F);
  if (p.R > 0) {
    if (p.f32)
      hipLaunchKernelGGL((k_gather<float, false>), dim3(p.max_tiles), dim3(256), 0, st, F);
    else
      hipLaunchKernelGGL((k_gather<bf16_t, false>), dim3(p.max_tiles), dim3(256), 0, st, F);
  }
  return launch_status();
}

int moe_gather(const moe_desc* desc, const void* x, const int32_t* perm, const int32_t* inv, void* xp,
               uint8_t* xp_scale, void* stream) {
  Plan p;
  int rc = make_plan(desc, &p);
  if (rc != MOE_OK) return rc;
  if (p.macro) return MOE_ERR_UNSUPPORTED;
  if (p.R == 0) return MOE_OK;
  if (!x || (!perm && !inv) || !xp) return MOE_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)stream;
  if (p.mxfp8) {
    if (!xp_scale) return MOE_ERR_INVALID_ARG;
    return inv ? mxfp8_gather_push((const bf16_t*)x, inv, (uint8_t*)xp, xp_scale, p.T, p.R, p.d, p.k, st)
               : mxfp8_gather_perm((const bf16_t*)x, perm, (uint8_t*)xp, xp_scale, p.R, p.d, p.k, st);
  }
  if (inv) {
    const int grid = cdiv(p.T, 4) < 4096 ? cdiv(p.T, 4) : 4096;
    if (p.f32)
      hipLaunchKernelGGL(k_gather_push<float>, dim3(grid), dim3(256), 0, st, (const float*)x, inv, (float*)xp, p.T,
                         p.R, p.d, p.k);
    else
      hipLaunchKernelGGL(k_gather_push<bf16_t>, dim3(grid), dim3(256), 0, st, (const bf16_t*)x, inv, (bf16_t*)xp,
                         p.T, p.R, p.d, p.k);
    return launch_status();
  }
  const int grid = cdiv(p.R, 4) < 4096 ? cdiv(p.R, 4) : 4096;
  if (p.f32)
    hipLaunchKernelGGL(k_gather_perm<float>, dim3(grid), dim3(256), 0, st, (const float*)x, perm, (float*)xp, p.R,
                       p.d, p.k);
  else
    hipLaunchKernelGGL(k_gather_perm<bf16_t>, dim3(grid), dim3(256), 0, st, (const bf16_t*)x, perm, (bf16_t*)xp,
                       p.R, p.d, p.k);
  return launch_status();
}

int moe_combine(const moe_desc* desc, const void* yp, const float* gate, const int32_t* inv, void* y,
                void* stream) {
  Plan p;
  int rc = make_plan(desc, &p, true);
  if (rc != MOE_OK) return rc;
  if (p.macro) return MOE_ERR_UNSUPPORTED;
  if (p.T == 0) return MOE_OK;
  if (!yp || !gate || !inv || !y) return MOE_ERR_INVALID_ARG;
  Fwd F;
  memset(&F, 0, sizeof(F));
  F.T = p.T; F.d = p.d; F.k = p.k; F.R = p.R; F.E = p.E;
  F.yp = const_cast<void*>(yp);
  F.gate = const_cast<float*>(gate);
  F.inv = const_cast<int32_t*>(inv);
  F.y = y;
  hipStream_t st = (hipStream_t)stream;
  if (p.f32)
    hipLaunchKernelGGL(k_combine_alone<float>, dim3(p.nC), dim3(256), 0, st, F);
  else
    hipLaunchKernelGGL(k_combine_alone<bf16_t>, dim3(p.nC), dim3(256), 0, st, F);
  return launch_status();
}

int moe_quantize_mxfp8(const void* src, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales, void* stream) {
  if (rows < 0 || K <= 0 || K % 32) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;
  if (!src || !codes || !scales) return MOE_ERR_INVALID_ARG;
  return mxfp8_quantize_rows((const bf16_t*)src, rows, K, codes, scales, (hipStream_t)stream);
}

int moe_quantize_mxfp8_t(const void* src, int64_t batch, int64_t rows, int64_t cols, uint8_t* codes,
                         uint8_t* scales, void* stream) {
  if (batch < 0 || rows <= 0 || cols <= 0 || rows % 32) return MOE_ERR_INVALID_ARG;
  if (batch > 65535 || cdiv64(rows, 128) > 65535 || cols > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
  if (batch == 0) return MOE_OK;
  if (!src || !codes || !scales) return MOE_ERR_INVALID_ARG;
  const dim3 grid((unsigned)cdiv((int)cols, 128), (unsigned)cdiv((int)rows, 128), (unsigned)batch);
  if (cols % 8 == 0 && ((uintptr_t)src & 15) == 0)
    hipLaunchKernelGGL(k_mx_quant_t<true>, grid, dim3(kThreads), 0, (hipStream_t)stream, (const bf16_t*)src, codes,
                       scales, (int)rows, (int)cols);
  else
    hipLaunchKernelGGL(k_mx_quant_t<false>, grid, dim3(kThreads), 0, (hipStream_t)stream, (const bf16_t*)src, codes,
                       scales, (int)rows, (int)cols);
  return launch_status();
}

static Fwd forward_args(const Plan& p, const moe_desc* desc, const void* x, const void* wr, const float* bias,
                        const moe_weights* w, void* y, const moe_saved* saved, void* workspace) {
  Fwd F = make_fwd(p, desc, workspace, saved);
  F.x = x; F.wr = wr; F.bias = bias; F.w1 = w->w1; F.w3 = w->w3; F.w2 = w->w2; F.y = y;
  if (p.mxfp8) {
    F.w1s = w->w1_scale; F.w3s = w->w3_scale; F.w2s = w->w2_scale;
    auto al16 = [](const void* q) { return ((uintptr_t)q & 15) == 0; };
    F.mx_wide1 = p.d % 512 == 0 && al16(F.xs) && al16(F.w1s) && al16(F.w3s);
    F.mx_wide2 = p.I % 512 == 0 && al16(F.hs) && al16(F.w2s);
  }
  return F;
}

static int forward_run(const Plan& p, const moe_desc* desc, const Fwd& F, hipStream_t st, bool ring = false) {
  if (p.mxfp8) return forward_impl<bf16_t, TileMX128>(p, desc, F, st, ring);
  if (p.f32) return forward_impl<float, TileB128>(p, desc, F, st, ring);
  if (p.BM == 256) return forward_impl<bf16_t, TileD256w>(p, desc, F, st, ring);
  if (p.BM == 64) return forward_impl<bf16_t, TileD256h>(p, desc, F, st, ring);
  return forward_impl<bf16_t, TileD256>(p, desc, F, st, ring);
}

static int forward_call(const Plan& p, const moe_desc* desc, const void* x, const void* wr, const float* bias,
                        const moe_weights* w, void* y, const moe_saved* saved, void* workspace, hipStream_t st) {
  return forward_run(p, desc, forward_args(p, desc, x, wr, bias, w, y, saved, workspace), st);
}

// Bytes of one slot of the macrobatch ring: the forward's regions for Tm
// tokens (0 for an invalid descriptor).
static size_t forward_bytes(const moe_desc* desc, int T);
static size_t ring_slot_bytes(const moe_desc* desc, int Tm) { return align256(forward_bytes(desc, Tm)); }

// Macrobatches (MoK flash §02: token volume streamed through a fixed ring
// of token buffers): the forward over consecutive ranges of Tm tokens (the
// last one ragged) through a ring of two workspace slots, macrobatch i in
// slot i % 2.  With the persistent path, the launch of macrobatch i also
// runs the merge of macrobatch i-1 -- whose expert outputs sit in the other
// slot, complete at the launch boundary -- as extra tasks of its first
// phase, so that merge overlaps this macrobatch's routing and dispatch; the
// last macrobatch's merge follows as a plain launch.  A slot is written
// again two launches later, after the launch that merged from it has ended
// (stream order), so every buffer is written once per launch as in a single
// call.  Per-token outputs only (no layout over all tokens).
static int forward_in_batches(const moe_desc* desc, int Tm, const void* x, const void* wr, const float* bias,
                              const moe_weights* w, void* y, const moe_saved* saved, void* workspace,
                              hipStream_t st) {
  const int T = desc->T, E = desc->E, k = desc->k, d = desc->d;
  const size_t es = desc->act_dtype == MOE_F32 ? 4 : 2;
  const size_t slot = ring_slot_bytes(desc, Tm);
  const bool ring = desc->fused != 0;
  Fwd prev;
  bool have_prev = false;
  bool prev_f32 = false;
  for (int t0 = 0, i = 0; t0 < T; t0 += Tm, ++i) {
    moe_desc md = *desc;
    md.T = T - t0 < Tm ? T - t0 : Tm;
    md.macro_tokens = 0;
    Plan pm;
    int rc = make_plan(&md, &pm, true);  // the forward's regions only
    if (rc != MOE_OK) return rc;
    moe_saved sm;
    memset(&sm, 0, sizeof(sm));
    if (saved) {
      sm.logits = saved->logits ? saved->logits + (size_t)t0 * E : nullptr;
      sm.topk_idx = saved->topk_idx ? saved->topk_idx + (size_t)t0 * k : nullptr;
      sm.gate = saved->gate ? saved->gate + (size_t)t0 * k : nullptr;
      sm.status = saved->status;
    }
    void* ws = (char*)workspace + (size_t)(i & 1) * slot;
    Fwd F = forward_args(pm, &md, (const char*)x + (size_t)t0 * d * es, wr, bias, w,
                         (char*)y + (size_t)t0 * d * es, saved ? &sm : nullptr, ws);
    if (ring && have_prev) {
      F.prev = Merge{prev.T, prev.d, prev.k, prev.R, prev.yp, prev.gate, prev.inv, prev.y};
      F.prev_nC = prev.nC;
      F.prev_abort = prev.s.abort;
    }
    rc = forward_run(pm, &md, F, st, ring);
    if (rc != MOE_OK) return rc;
    prev = F;
    prev_f32 = pm.f32;
    have_prev = pm.T > 0;
  }
  if (ring && have_prev) {
    if (prev_f32)
      hipLaunchKernelGGL(k_combine<float>, dim3(prev.nC), dim3(256), 0, st, prev);
    else
      hipLaunchKernelGGL(k_combine<bf16_t>, dim3(prev.nC), dim3(256), 0, st, prev);
    return launch_status();
  }
  return MOE_OK;
}

// ------------------------------------------------------------------ no-alloc
// The forward's workspace in a static device array, for callers that cannot
// allocate.  Each device the library runs on holds its own copy until the
// process ends; host code reaches it only through the address
// hipGetSymbolAddress gives on that device (the array's name is a host-side
// stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static void* g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// The scratch array's device address on the current device, looked up once
// per device with that device current.
static int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Forward workspace bytes of T tokens, or 0 for an invalid descriptor.
static size_t forward_bytes(const moe_desc* desc, int T) {
  moe_desc md = *desc;
  md.T = T;
  md.macro_tokens = 0;
  Plan q;
  return make_plan(&md, &q, true) == MOE_OK ? q.total : 0;
}

int moe_forward(const moe_desc* desc, const void* x, const void* wr, const float* bias, const moe_weights* w,
                void* y, const moe_saved* saved, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  int rc = make_plan(desc, &p);
  if (rc != MOE_OK) return rc;
  if (!w || (p.T > 0 && (!x || !wr || !y || !w->w1 || !w->w3 || !w->w2))) return MOE_ERR_INVALID_ARG;
  if (p.mxfp8 && (!w->w1_scale || !w->w3_scale || !w->w2_scale)) return MOE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < p.total) return MOE_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  if (!p.macro) return forward_call(p, desc, x, wr, bias, w, y, saved, workspace, st);
  if (saved && (saved->counts || saved->offsets || saved->perm || saved->inv || saved->a || saved->b || saved->h))
    return MOE_ERR_INVALID_ARG;
  return forward_in_batches(desc, p.T, x, wr, bias, w, y, saved, workspace, st);
}

int moe_forward_noalloc(const moe_desc* desc, const void* x, const void* wr, const float* bias,
                        const moe_weights* w, void* y, const moe_saved* saved, void* stream) {
  Plan p;
  int rc = make_plan(desc, &p, true);
  if (rc != MOE_OK) return rc;
  if (!w || (p.T > 0 && (!x || !wr || !y || !w->w1 || !w->w3 || !w->w2))) return MOE_ERR_INVALID_ARG;
  if (p.mxfp8 && (!w->w1_scale || !w->w3_scale || !w->w2_scale)) return MOE_ERR_INVALID_ARG;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != MOE_OK) return rc;
  hipStream_t st = (hipStream_t)stream;
  // tokens per call: all of them when their workspace fits (and the caller
  // asked for no macrobatches), else macrobatches of the most tokens whose
  // two ring slots fit, at most macro_tokens
  const int T = desc->T;
  const size_t all = forward_bytes(desc, T);
  int Tm = T;
  if (p.macro || all == 0 || all > MOE_NOALLOC_SCRATCH_BYTES) {
    const int cap = p.macro ? p.T : T;
    auto fits = [&](int n) {
      const size_t b = forward_bytes(desc, n);
      return b != 0 && 2 * ring_slot_bytes(desc, n) <= MOE_NOALLOC_SCRATCH_BYTES;
    };
    int lo = 0, hi = cap + 1;  // largest fitting count in [lo, hi)
    while (hi - lo > 1) {
      const int mid = lo + (hi - lo) / 2;
      if (fits(mid)) lo = mid; else hi = mid;
    }
    Tm = lo;
    if (T > 0 && Tm < 1) return MOE_ERR_WORKSPACE;  // not one token's ring fits
  }
  if (Tm >= T) {
    moe_desc md = *desc;
    md.macro_tokens = 0;
    Plan pf;
    rc = make_plan(&md, &pf, true);
    if (rc != MOE_OK) return rc;
    return forward_call(pf, &md, x, wr, bias, w, y, saved, ws, st);
  }
  // the layout and the saved activations describe one batch over all T
  if (saved && (saved->counts || saved->offsets || saved->perm || saved->inv || saved->a || saved->b || saved->h))
    return MOE_ERR_WORKSPACE;
  return forward_in_batches(desc, Tm, x, wr, bias, w, y, saved, ws, st);
}

int moe_backward(const moe_desc* desc, const void* dy, const void* x, const moe_weights* w, const moe_saved* saved,
                 void* dx, void* dw1, void* dw3, void* dw2, float* dgate, void* workspace, size_t workspace_bytes,
                 void* stream) {
  Plan p;
  int rc = make_plan(desc, &p);
  if (rc != MOE_OK) return rc;
  if (p.macro) return MOE_ERR_UNSUPPORTED;
  if (!p.bwd_ok) return MOE_ERR_UNSUPPORTED;
  if (!w || !saved) return MOE_ERR_INVALID_ARG;
  if (!saved->offsets || !dw1 || !dw3 || !dw2 || !w->w1 || !w->w3 || !w->w2) return MOE_ERR_INVALID_ARG;
  if (p.mxfp8 && (!w->w1_scale || !w->w3_scale || !w->w2_scale)) return MOE_ERR_INVALID_ARG;
  if (p.T > 0 && (!dy || !x || !dx || !dgate || !saved->gate || !saved->perm || !saved->inv || !saved->a ||
                  !saved->b || !saved->h))
    return MOE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < p.total) return MOE_ERR_WORKSPACE;
  return backward_impl(p, desc, dy, x, w, saved, dx, dw1, dw3, dw2, dgate, workspace, (hipStream_t)stream);
}

int moe_router_backward(const moe_desc* desc, const void* x, const void* wr, const float* bias,
                        const moe_saved* saved, const float* dgate, float* dlogits, void* dwr, float* dbias,
                        void* dx, void* workspace, size_t workspace_bytes, void* stream) {
  Plan p;
  int rc = make_plan(desc, &p);
  if (rc != MOE_OK) return rc;
  if (p.macro) return MOE_ERR_UNSUPPORTED;
  if (desc->score == MOE_SCORE_SOFTMAX && !desc->renorm) return MOE_ERR_UNSUPPORTED;
  if (!saved || !wr || !dwr || !saved->offsets) return MOE_ERR_INVALID_ARG;
  if (p.T > 0 && (!x || !dx || !dgate || !saved->logits || !saved->topk_idx || !saved->gate || !saved->perm))
    return MOE_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < p.total) return MOE_ERR_WORKSPACE;
  RouterBwd P;
  memset(&P, 0, sizeof(P));
  P.T = p.T; P.d = p.d; P.E = p.E; P.k = p.k; P.R = p.R;
  P.score = desc->score; P.renorm = desc->renorm ? 1 : 0;
  P.select_only = (desc->flags & MOE_FLAG_BIAS_SELECT_ONLY) ? 1 : 0;
  P.scale = desc->routed_scale > 0.0f ? desc->routed_scale : 1.0f;
  P.x = x; P.wr = wr; P.bias = bias; P.logits = saved->logits; P.topk = saved->topk_idx;
  P.gate = saved->gate; P.dgate = dgate; P.offsets = saved->offsets; P.perm = saved->perm;
  P.dz = at<float>(workspace, p.o_rdz);
  P.part = at<float>(workspace, p.o_rpart);
  P.pbias = at<float>(workspace, p.o_rpbias);
  P.dlogits = dlogits; P.dwr = dwr; P.dbias = dbias; P.dx = dx;
  hipStream_t st = (hipStream_t)stream;
  const int nvec = p.d * p.act_es / 16;
  const int tgrid = cdiv(p.T, 4) < 4096 ? cdiv(p.T, 4) : 4096;
  const int64_t nel = (int64_t)p.E * p.d;
  const int fgrid = (int)(cdiv64(nel, 256) < 8192 ? cdiv64(nel, 256) : 8192);
  const dim3 wgrid(p.E, cdiv(nvec, 64), kRbSplits);
  if (p.f32) {
    if (p.T > 0) hipLaunchKernelGGL(k_router_bwd_tokens<float>, dim3(tgrid), dim3(256), 0, st, P);
    hipLaunchKernelGGL(k_router_bwd_dwr<float>, wgrid, dim3(256), 0, st, P);
    hipLaunchKernelGGL(k_router_bwd_final<float>, dim3(fgrid), dim3(256), 0, st, P);
  } else {
    if (p.T > 0) hipLaunchKernelGGL(k_router_bwd_tokens<bf16_t>, dim3(tgrid), dim3(256), 0, st, P);
    hipLaunchKernelGGL(k_router_bwd_dwr<bf16_t>, wgrid, dim3(256), 0, st, P);
    hipLaunchKernelGGL(k_router_bwd_final<bf16_t>, dim3(fgrid), dim3(256), 0, st, P);
  }
  return launch_status();
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid argument";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: shape or type combination not supported";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch failed";
    case MOE_ERR_TIMEOUT: return "MOE_ERR_TIMEOUT: a device-side wait exceeded its bound";
    case MOE_ERR_INVALID_ROUTE: return "MOE_ERR_INVALID_ROUTE: expert index out of range or repeated";
    default: return "unknown moe_status";
  }
}

}  // extern "C"
