// protocol.h -- the task-claiming and waiting protocol of the persistent
// kernels, written once for the device and for a host model of it (a
// std::thread program that runs it under ThreadSanitizer).
//
// MoK flash (the page "Cursor's MoK achieves 2.37x performance boost on
// NVIDIA GB300 NVL72"), §02: inside one kernel the side that stages tokens
// tells the expert side through GPU-local counters that a batch is complete;
// §01: compute may not start before its data is complete and visible.
//
// The includer defines MOE_PROTO_FN (the function qualifiers: device or
// host) and supplies an Ops policy with
//   int  load(const int* p)             coherent load of a counter
//   int  fetch_add(int* p, int v)       atomic add, returns the old value
//   void store(int* p, int v)           coherent store
//   void set_status(int32_t* s, int c)  first error wins (s may be null)
//   void pause()                        back off between polls
//
// Claiming.  The tasks of a call form phases; a task only ever waits on
// tasks of earlier phases.  Each phase is split into kXcds sub-queues: group
// g of a phase belongs to sub-queue g % kXcds.  A worker drains its own
// sub-queue of the current phase, then the other ones, and only then moves
// to the next phase; so when any task of phase p+1 is claimed, every task of
// phase p has been claimed by a running worker, and by induction over the
// phases every wait ends whatever the number of workers and whichever
// sub-queue each starts on (that only steers locality).
//
// Waiting.  Every wait is bounded.  A task whose wait failed neither runs
// nor raises its own counter, so no count ever covers work that was not
// done, and a wait that finds its count met may proceed.  A poll that finds
// it short reads the abort word: once any wait has given up (and raised
// abort) every wait still short fails at its next poll and the workers
// drain the queues without doing dependent work.  (Reading abort on a poll
// that found the count met would put a second serial agent-scope load on
// every task; on the MXFP8 down projection that cost a quarter of its time.)
#pragma once

#include <stdint.h>

#ifndef MOE_PROTO_FN
#error "define MOE_PROTO_FN (the function qualifiers) before including protocol.h"
#endif

namespace moe {
namespace proto {

constexpr int kMaxPhases = 8;
constexpr int kXcds = 8;
constexpr int kErrTimeout = -5;  // MOE_ERR_TIMEOUT

// Claim state of one worker.
struct Claim {
  int phase;  // current phase
  int qoff;   // sub-queue being drained: (own + qoff) % kXcds
  int own;    // the worker's home sub-queue (its XCD)
  int nmt;    // row tiles once known, else -1
  int task;   // the claimed task (-1: done)
};

MOE_PROTO_FN void claim_advance(Claim& c) {
  if (++c.qoff == kXcds) {
    c.qoff = 0;
    ++c.phase;
  }
}

// shape(phase, groups, per) gives the phase's group count and tasks per
// group (it may wait; false = give up).  Returns the claimed task's index
// within its phase (group * per + member) and sets c.phase, or -1 when
// every phase is drained or shape gave up.  (Issuing a worker's next claim
// while its current task runs was measured slower: a task claimed early
// starts late, and the counters others wait on rise late with it.)
template <class Ops, class F>
MOE_PROTO_FN int claim_next(int* qctr, int nphases, Claim& c, F shape) {
  while (c.phase < nphases) {
    int groups = 0, per = 0;
    if (!shape(c.phase, groups, per)) return -1;
    const int sub = (c.own + c.qoff) & (kXcds - 1);
    const int g_sub = groups > sub ? (groups - sub + kXcds - 1) / kXcds : 0;
    const int n = g_sub * per;
    if (n > 0) {
      const int i = Ops::fetch_add(&qctr[c.phase * kXcds + sub], 1);
      if (i < n) return (sub + kXcds * (i / per)) * per + i % per;
    }
    claim_advance(c);
  }
  return -1;
}

struct WaitCtx {
  int* abort;
  int32_t* status;
  long long spin_limit;
};

// True once *ctr >= target, false when abort is (or becomes) set or after
// spin_limit polls (then MOE_ERR_TIMEOUT is recorded and abort raised).
template <class Ops>
MOE_PROTO_FN bool wait_geq(const int* ctr, int target, const WaitCtx& w) {
  for (long long spins = 0;; ++spins) {
    if (Ops::load(ctr) >= target) return true;
    if (Ops::load(w.abort)) return false;
    if (spins >= w.spin_limit) {
      Ops::set_status(w.status, kErrTimeout);
      Ops::store(w.abort, 1);
      return false;
    }
    Ops::pause();
  }
}

}  // namespace proto
}  // namespace moe
