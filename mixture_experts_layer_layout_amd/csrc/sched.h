// sched.h -- task claiming for the persistent kernels.
//
// The tasks of a layer call form phases (routing, top-k, layout, gather,
// up-projection tiles, ...); a task only ever waits on tasks of earlier
// phases.  Each phase is split into 8 sub-queues, one per XCD: the tasks of
// a phase come in groups (a row tile's column tiles, an expert's weight
// gradient tiles) and group g belongs to sub-queue g % 8, so the tasks that
// share an operand run on one XCD and share its L2.  A workgroup drains its
// own XCD's sub-queue of the current phase, then the other seven, and only
// then moves to the next phase.  Hence when any task of phase p+1 is claimed
// every task of phase p has already been claimed by a running workgroup;
// by induction over phases every wait ends, whatever the grid size and
// whichever XCD each workgroup lands on (the XCD only steers locality).
#pragma once

#include "common.h"

namespace moe {

using proto::kMaxPhases;
using proto::kXcds;
using proto::Claim;

// The XCD this wave runs on (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ int xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (kXcds - 1);
}

// The home sub-queue of this workgroup: its XCD, or (the test-only
// MOE_FLAG_TEST_SHUFFLE_CLAIMS) a hash of its workgroup id, which changes the
// order in which the tasks are claimed and where they run without changing
// what any task computes.
__device__ __forceinline__ int claim_home(uint32_t flags) {
  if (flags & MOE_FLAG_TEST_SHUFFLE_CLAIMS) return (int)((blockIdx.x * 0x9E3779B1u) >> 29);
  return xcc_id();
}

// Thread 0 only (protocol.h: claim_next).
template <class F>
__device__ __forceinline__ int claim_next(int* qctr, int nphases, Claim& c, F shape) {
  return proto::claim_next<DevOps>(qctr, nphases, c, shape);
}

// ---------------------------------------------------------------- raster
// Tasks per block of the grouped raster: about one XCD's worth of
// concurrently resident workgroups (32 CUs x 2).
constexpr int kRasterBlock = 64;

// Task i of a phase over the (row tile, column tile) grid of every expert
// -> (tile, nt).  Expert e owns row tiles [etile[e], etile[e+1]) and tasks
// [etile[e] * NT, etile[e+1] * NT).  Each expert's grid is walked in blocks
// of at most 8 row tiles x (64 / rows) column tiles, row tile fastest, so
// the kRasterBlock consecutive tasks that one XCD runs together share their
// activation rows and weight columns in that XCD's L2.
__device__ __forceinline__ void raster_decode(const int* etile, int E, int NT, int i, int& tile, int& nt) {
  const int q = i / NT;
  int lo = 0, hi = E;  // the last expert with etile[e] <= q
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (etile[mid] <= q) lo = mid; else hi = mid;
  }
  const int base = etile[lo], MT = etile[lo + 1] - base;
  int j = i - base * NT;
  const int RG = min(MT, 8);
  const int band = j / (RG * NT);
  j -= band * RG * NT;
  const int h = min(RG, MT - band * RG);
  const int CG = min(NT, max(1, kRasterBlock / h));
  const int cg = j / (h * CG);
  j -= cg * h * CG;
  tile = base + band * RG + j % h;
  nt = cg * CG + j / h;
}

}  // namespace moe
