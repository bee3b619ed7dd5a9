// plan.h -- host-side validation of a layer description and the carving of
// one caller-owned workspace into the buffers the kernels use.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

struct Plan {
  int T, d, E, k, I, R;  // T: tokens of one call (of one macrobatch when macro)
  bool macro;      // moe_forward runs macrobatches of T tokens over T_full
  int T_full;
  int nb;          // token blocks of 64
  int S;           // router k-slices
  int BM;          // rows per row tile (= rows per ready counter)
  int nN1, nN2;    // column tiles of the up / down projection
  int nC;          // combine tasks
  int max_tiles;   // upper bound on row tiles: R/BM + min(E, R)
  int act_es;      // bytes per activation element
  bool f32, mxfp8;
  // backward (bf16; needs d % 128 == 0 and I % 128 == 0)
  bool bwd_ok;
  int nNdh;        // column tiles of the dH GEMM (over I)
  int nNdx;        // column tiles of the dXp GEMM (over d)
  int nW2m, nW2n;  // dW2 tiles per expert: over d, over I
  int nW13m, nW13n;// dW1/dW3 tiles per expert: over I (half a tile of each), over d
  int nRP;         // row-preparation tasks (kPrepTok tokens each)
  // workspace carving (byte offsets)
  size_t o_ctr, n_ctr;
  size_t lstride;  // floats per router slice (T E rounded up to 32)
  size_t o_lpart, o_topk, o_gate, o_bmask, o_bbase, o_counts, o_offsets;
  size_t o_tile_e, o_tile_r0, o_tile_n, o_perm, o_inv, o_src, o_grow;
  size_t o_etile, o_eorder, o_eoff, o_tsrc;
  size_t o_h, o_big1, o_big2, o_dab, o_dgp, o_hs, o_zero, o_gg;
  size_t o_xs;     // MXFP8: x scales (the codes sit at o_big1)
  size_t o_rdz, o_rpart, o_rpbias;  // router backward: dz, dWr and dbias partial sums
  size_t o_dyq, o_dys, o_dabq, o_dabs;  // MXFP8 backward: dY and [dA | dB] codes and scales
  bool mx_wgrad;   // MXFP8 backward with MXFP8 weight gradients (MOE_FLAG_MXFP8_WGRAD)
  int kcap;        // then: row-tile slots of the weight gradients' operands (max_tiles * 128)
  size_t o_xT, o_xTs, o_gT, o_gTs, o_hT, o_hTs, o_dabT, o_dabTs;  // their codes and scales
  size_t total;
};

// Counter region, in ints.
enum CtrSlot {
  C_QUEUE = 0, C_ABORT, C_R2, C_SCAN, C_G2, C_NMT, C_AUX3, C_QDONE, C_HEADER = 16
};

// fwd_only: carve only the regions the forward uses (moe_forward_noalloc)
int make_plan(const moe_desc* d, Plan* p, bool fwd_only = false);

}  // namespace moe
