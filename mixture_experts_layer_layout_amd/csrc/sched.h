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

constexpr int kMaxPhases = 8;
constexpr int kXcds = 8;

// The XCD this wave runs on (hardware register XCC_ID, bits 3:0).
__device__ __forceinline__ int xcc_id() {
  return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & (kXcds - 1);
}

// Claim state of one workgroup, kept in LDS (only thread 0 touches it) so
// it occupies no registers across the tasks of the persistent loop.
struct Claim {
  int phase;  // current phase
  int qoff;   // sub-queue being drained: (own + qoff) % 8
  int own;    // this workgroup's XCD
  int nmt;    // row tiles once known, else -1
  int task;   // the claimed task (-1: done)
};

// Thread 0 only.  shape(phase, groups, per) gives the phase's group count
// and tasks per group (it may wait for the layout; false = give up).
// Returns the claimed task's index within its phase (group * per + member)
// and sets c.phase, or returns -1 when every phase is drained.
template <class F>
__device__ __forceinline__ int claim_next(int* qctr, int nphases, Claim& c, F shape) {
  while (c.phase < nphases) {
    int groups = 0, per = 0;
    if (!shape(c.phase, groups, per)) return -1;
    const int sub = (c.own + c.qoff) & (kXcds - 1);
    const int g_sub = groups > sub ? (groups - sub + kXcds - 1) / kXcds : 0;
    const int n = g_sub * per;
    if (n > 0) {
      const int i = atomicAdd(&qctr[c.phase * kXcds + sub], 1);
      if (i < n) return (sub + kXcds * (i / per)) * per + i % per;
    }
    if (++c.qoff == kXcds) {
      c.qoff = 0;
      ++c.phase;
    }
  }
  return -1;
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
