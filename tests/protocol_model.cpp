// protocol_model.cpp -- a host model of the persistent kernels' task
// protocol, built with -fsanitize=thread by tests/test_protocol_model.py.
//
// Test infrastructure.  Workgroups are std::threads; the claiming and the
// bounded waits are the device's own code (csrc/protocol.h), compiled here
// with host atomics; the phases, what each task waits for and what it
// raises, mirror the persistent forward (moe.hip: k_fused_fwd) and backward
// (k_fused_bwd), each launch a set of threads joined before the next (the
// kernel boundary).  Every task writes the data it produces with plain
// stores and checks, with plain loads, that the data it consumes holds the
// producer's value; ThreadSanitizer reports any such access that no
// counter orders after its producer, and a wrong value counts as a
// violation.
//
// MoK flash (the page "Cursor's MoK achieves 2.37x performance boost on
// NVIDIA GB300 NVL72"), §02: the staging side tells the expert side through
// GPU-local counters that a batch is complete; §01: compute may not start
// before its data is complete.
//
// Built with -DPLANT_NO_READY_WAIT or -DPLANT_RUN_AFTER_FAILED_WAIT it plants
// a mistake in the model (the test checks that the model then fails).
//
// usage: protocol_model <scenario> <workers> <seed>
//   scenarios: fwd-single, fwd-default, fwd-drop, fwd-tiny, bwd-single,
//              bwd-default
//   prints "ok status=<s> tasks=<n>" and exits 0, or reports and exits 1
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <functional>
#include <random>
#include <string>
#include <thread>
#include <vector>

#define MOE_PROTO_FN inline
#include "../mixture_experts_layer_layout_amd/csrc/protocol.h"

using moe::proto::Claim;
using moe::proto::kXcds;
using moe::proto::WaitCtx;

// The orderings the device provides: claims, the abort word and the status
// are relaxed atomics (they order nothing); a counter is raised with a
// release (the producer's agent-scope release before its atomic add) and
// polled with an acquire (the consumer's poll and workgroup acquire after
// it).  So the only happens-before edges between tasks are the counters.
struct HostOps {
  static int load(const int* p) { return __atomic_load_n(p, __ATOMIC_ACQUIRE); }
  static int fetch_add(int* p, int v) { return __atomic_fetch_add(p, v, __ATOMIC_RELAXED); }
  static void store(int* p, int v) { __atomic_store_n(p, v, __ATOMIC_RELAXED); }
  static void set_status(int32_t* s, int c) {
    if (!s) return;
    int32_t z = 0;
    __atomic_compare_exchange_n(s, &z, c, false, __ATOMIC_RELAXED, __ATOMIC_RELAXED);
  }
  static void pause() { std::this_thread::yield(); }
};

static void signal(int* ctr) { __atomic_fetch_add(ctr, 1, __ATOMIC_RELEASE); }

// Random delays inside tasks, so that producers and consumers really overlap
// (under the sanitizer a worker that starts first would otherwise drain
// most of the queue alone).
static thread_local std::mt19937_64 t_rng{12345};
static void jitter() {
  const uint64_t r = t_rng() % 8;
  if (r < 3) std::this_thread::sleep_for(std::chrono::microseconds(t_rng() % 60));
  else if (r < 6) std::this_thread::yield();
}

static std::atomic<long> g_violations{0};
static std::atomic<long> g_tasks{0};

static void check(bool ok, const char* what, int a, int b) {
  if (!ok) {
    if (g_violations.fetch_add(1) < 10) fprintf(stderr, "violation: %s (%d, %d)\n", what, a, b);
  }
}

// One persistent launch: `workers` threads claim tasks of the phases in
// `mask` through claim_next and run body(phase, task) until drained.
// shape(phase, groups, per, claim) as on the device.
struct Launch {
  int nphases;
  unsigned mask;
  std::function<bool(int, int&, int&, Claim&)> shape;
  std::function<void(int, int, const Claim&)> body;
};

static void run_launch(int* qctr, const Launch& L, int workers, uint64_t seed) {
  std::vector<std::thread> th;
  std::atomic<int> started{0};
  for (int w = 0; w < workers; ++w) {
    th.emplace_back([&, w] {
      std::mt19937_64 rng(seed * 1000003u + w);
      t_rng.seed(seed * 7919u + w);
      // every worker starts claiming together (the barrier orders no task)
      started.fetch_add(1, std::memory_order_relaxed);
      while (started.load(std::memory_order_relaxed) < workers) std::this_thread::yield();
      Claim c;
      c.phase = 0;
      c.qoff = 0;
      c.own = (int)(rng() % kXcds);  // a random home sub-queue: any claim order
      c.nmt = -1;
      for (;;) {
        auto shape = [&](int ph, int& groups, int& per) -> bool {
          per = 1;
          groups = 0;
          if (!((L.mask >> ph) & 1u)) return true;
          return L.shape(ph, groups, per, c);
        };
        const int t = moe::proto::claim_next<HostOps>(qctr, L.nphases, c, shape);
        if (t < 0) break;
        jitter();
        L.body(c.phase, t, c);
        g_tasks.fetch_add(1, std::memory_order_relaxed);
      }
    });
  }
  for (auto& t : th) t.join();
}

// ---------------------------------------------------------------- forward
// Phases (k_fused_fwd): 0 router slices (nb * S), 1 top-k (nb * C), 2 layout
// scan (1), 3 gather (ntiles), 4 up projection (ntiles * N1), 5 down
// projection (ntiles * N2), 6 combine (NC).  Waits: top-k on r1[b] >= S,
// scan on r2 >= nb C, phases >= 3 on scan_done >= 1 (in the claim), up
// projection on ready[tile] >= 1, down projection on hcnt[tile] >= N1,
// combine on g2 >= ntiles N2.
struct FwdModel {
  int nb = 5, S = 3, C = 4, N1 = 3, N2 = 2, NC = 6;
  int ntiles_true = 0;  // decided by the scan
  int drop_tile = -1;   // gather of this tile raises no counter
  // counters
  std::vector<int> qctr, r1, ready, hcnt;
  int r2 = 0, scan_done = 0, g2 = 0, n_mtiles = 0, abort_ = 0;
  int32_t status = 0;
  long long spin;
  // data (plain)
  std::vector<int> lpart, topk, tile_rows, tsrc, h, yp, y;
  std::vector<int> ran_up;  // an up-projection task of a tile ran (atomic flag)
  int max_tiles = 64;

  explicit FwdModel(long long spin_limit, uint64_t seed) : spin(spin_limit) {
    std::mt19937_64 rng(seed);
    ntiles_true = 1 + (int)(rng() % 20);
    qctr.assign(moe::proto::kMaxPhases * kXcds, 0);
    r1.assign(nb, 0);
    ready.assign(max_tiles, 0);
    hcnt.assign(max_tiles, 0);
    lpart.assign(nb * S, -1);
    topk.assign(nb * C, -1);
    tile_rows.assign(max_tiles, -1);
    tsrc.assign(max_tiles, -1);
    h.assign(max_tiles * N1, -1);
    yp.assign(max_tiles * N2, -1);
    y.assign(NC, -1);
    ran_up.assign(max_tiles, 0);
  }
  WaitCtx W() { return WaitCtx{&abort_, &status, spin}; }
  bool wait(const int* ctr, int target) { return moe::proto::wait_geq<HostOps>(ctr, target, W()); }

  bool shape(int ph, int& groups, int& per, Claim& c) {
    if (ph == 0) { groups = nb * S; return true; }
    if (ph == 1) { groups = nb * C; return true; }
    if (ph == 2) { groups = 1; return true; }
    if (c.nmt < 0) {
      if (!wait(&scan_done, 1)) return false;
      c.nmt = HostOps::load(&n_mtiles);
    }
    if (ph == 3) { groups = c.nmt; return true; }
    if (ph == 4) { groups = c.nmt * N1; return true; }
    if (ph == 5) { groups = c.nmt * N2; return true; }
    groups = NC;
    return true;
  }

  void body(int ph, int t, const Claim& c) {
    if (ph == 0) {
      lpart[t] = 1000 + t;
      jitter();
      signal(&r1[t / S]);
    } else if (ph == 1) {
      const int b = t / C;
      if (!wait(&r1[b], S)) return;
      int sum = 0;
      for (int s = 0; s < S; ++s) {
        check(lpart[b * S + s] == 1000 + b * S + s, "top-k read a router slice not written", b, s);
        sum += lpart[b * S + s];
      }
      topk[t] = sum;
      signal(&r2);
    } else if (ph == 2) {
      if (!wait(&r2, nb * C)) return;
      for (int i = 0; i < nb * C; ++i) check(topk[i] >= 0, "scan read a top-k not written", i, 0);
      for (int i = 0; i < ntiles_true; ++i) tile_rows[i] = 100 + i;
      n_mtiles = ntiles_true;  // published by the release of scan_done
      signal(&scan_done);
    } else if (ph == 3) {
      if (t >= c.nmt) return;
      check(tile_rows[t] == 100 + t, "gather read a tile not listed", t, 0);
      jitter();
      tsrc[t] = 7000 + t;
      jitter();
      if (t == drop_tile) return;
      signal(&ready[t]);
    } else if (ph == 4) {
      if (t >= c.nmt * N1) return;
      const int tile = t / N1, nt = t % N1;
#if defined(PLANT_NO_READY_WAIT)
      // planted mistake: the up projection does not wait for its rows
#elif defined(PLANT_RUN_AFTER_FAILED_WAIT)
      // planted mistake: a task whose wait failed still runs
      wait(&ready[tile], 1);
#else
      if (!wait(&ready[tile], 1)) return;
#endif
      __atomic_store_n(&ran_up[tile], 1, __ATOMIC_RELAXED);  // bookkeeping only
      check(tsrc[tile] == 7000 + tile, "up projection read rows not staged", tile, nt);
      jitter();
      h[tile * N1 + nt] = 3 * tile + nt;
      signal(&hcnt[tile]);
    } else if (ph == 5) {
      if (t >= c.nmt * N2) return;
      const int tile = t / N2, nt = t % N2;
      if (!wait(&hcnt[tile], N1)) return;
      for (int j = 0; j < N1; ++j) check(h[tile * N1 + j] == 3 * tile + j, "down projection read H not written", tile, j);
      yp[tile * N2 + nt] = 5 * tile + nt;
      signal(&g2);
    } else if (ph == 6) {
      if (!wait(&g2, c.nmt * N2)) return;
      int sum = 0;
      for (int i = 0; i < c.nmt * N2; ++i) {
        check(yp[i] == 5 * (i / N2) + i % N2, "combine read a row not computed", i, 0);
        sum += yp[i];
      }
      y[t] = sum;
    }
  }

  Launch launch(unsigned mask) {
    Launch L;
    L.nphases = 7;
    L.mask = mask;
    L.shape = [this](int ph, int& g, int& p, Claim& c) { return shape(ph, g, p, c); };
    L.body = [this](int ph, int t, const Claim& c) { body(ph, t, c); };
    return L;
  }
  // a plain launch after the persistent ones (the combine kernel): skipped
  // when a wait of the call gave up
  void plain_combine() {
    if (HostOps::load(&abort_)) return;
    for (int t = 0; t < NC; ++t) {
      Claim c{};
      c.nmt = n_mtiles;
      int s = 0;
      for (int i = 0; i < c.nmt * N2; ++i) {
        check(yp[i] == 5 * (i / N2) + i % N2, "plain combine read a row not computed", i, 0);
        s += yp[i];
      }
      y[t] = s;
    }
  }
  bool complete() const {
    for (int i = 0; i < ntiles_true * N2; ++i)
      if (yp[i] != 5 * (i / N2) + i % N2) return false;
    for (int t = 0; t < NC; ++t)
      if (y[t] < 0) return false;
    return true;
  }
};

// ---------------------------------------------------------------- backward
// Phases (k_fused_bwd): 0 setup (1), 1 row preparation (NRP), 2 dh (ntiles *
// NDH), 3 dW2 (E bands), 4 dxp (ntiles * NDX), 5 dW1/dW3 (E bands), 6 dx
// (NC).  Waits: phases >= 2 on scan_done >= 1 + NRP (in the claim; dW2 and
// dW1/dW3 also in the task), dxp on hcnt[tile] >= NDH, dW1/dW3 of expert e
// on aux1[e] >= (tiles of e) NDH, dx on g2 >= ntiles NDX.
struct BwdModel {
  int E = 4, NRP = 5, NDH = 3, NDX = 2, NC = 5;
  std::vector<int> tiles_of;  // row tiles per expert
  int ntiles = 0;
  std::vector<int> qctr, hcnt, aux1;
  int scan_done = 0, g2 = 0, n_mtiles = 0, abort_ = 0;
  int32_t status = 0;
  long long spin;
  std::vector<int> tile_e, prep, dab, dxp, dw2, dw13, dx;

  BwdModel(long long spin_limit, uint64_t seed) : spin(spin_limit) {
    std::mt19937_64 rng(seed);
    for (int e = 0; e < E; ++e) tiles_of.push_back((int)(rng() % 4));  // experts may be empty
    for (int v : tiles_of) ntiles += v;
    qctr.assign(moe::proto::kMaxPhases * kXcds, 0);
    hcnt.assign(ntiles + 1, 0);
    aux1.assign(E, 0);
    tile_e.assign(ntiles + 1, -1);
    prep.assign(NRP, -1);
    dab.assign((ntiles + 1) * NDH, -1);
    dxp.assign((ntiles + 1) * NDX, -1);
    dw2.assign(E, -1);
    dw13.assign(E, -1);
    dx.assign(NC, -1);
  }
  WaitCtx W() { return WaitCtx{&abort_, &status, spin}; }
  bool wait(const int* ctr, int target) { return moe::proto::wait_geq<HostOps>(ctr, target, W()); }

  bool shape(int ph, int& groups, int& per, Claim& c) {
    if (ph == 0) { groups = 1; return true; }
    if (ph == 1) { groups = NRP; return true; }
    if (ph == 3 || ph == 5) { groups = E; return true; }
    if (c.nmt < 0) {
      if (!wait(&scan_done, 1 + NRP)) return false;
      c.nmt = HostOps::load(&n_mtiles);
    }
    if (ph == 2) { groups = c.nmt * NDH; return true; }
    if (ph == 4) { groups = c.nmt * NDX; return true; }
    groups = NC;
    return true;
  }
  void body(int ph, int t, const Claim& c) {
    if (ph == 0) {
      int id = 0;
      for (int e = 0; e < E; ++e)
        for (int i = 0; i < tiles_of[e]; ++i) tile_e[id++] = e;
      n_mtiles = ntiles;
      signal(&scan_done);
    } else if (ph == 1) {
      jitter();
      prep[t] = 40 + t;
      signal(&scan_done);
    } else if (ph == 3 || ph == 5) {
      if (!wait(&scan_done, 1 + NRP)) return;
      for (int i = 0; i < NRP; ++i) check(prep[i] == 40 + i, "weight gradient read rows not prepared", t, i);
      const int e = t;
      if (ph == 3) {
        dw2[e] = 1;
      } else {
        if (!wait(&aux1[e], tiles_of[e] * NDH)) return;
        int first = 0;
        for (int f = 0; f < e; ++f) first += tiles_of[f];
        for (int i = first; i < first + tiles_of[e]; ++i)
          for (int j = 0; j < NDH; ++j) check(dab[i * NDH + j] == i, "dW1/dW3 read dA|dB not written", i, j);
        dw13[e] = 1;
      }
    } else if (ph == 2) {
      if (t >= c.nmt * NDH) return;
      const int tile = t / NDH;
      check(tile_e[tile] >= 0, "dh read a tile not listed", tile, 0);
      for (int i = 0; i < NRP; ++i) check(prep[i] == 40 + i, "dh read rows not prepared", tile, i);
      jitter();
      dab[t] = tile;
      signal(&hcnt[tile]);
      signal(&aux1[tile_e[tile]]);
    } else if (ph == 4) {
      if (t >= c.nmt * NDX) return;
      const int tile = t / NDX;
      if (!wait(&hcnt[tile], NDH)) return;
      for (int j = 0; j < NDH; ++j) check(dab[tile * NDH + j] == tile, "dxp read dA|dB not written", tile, j);
      dxp[t] = tile;
      signal(&g2);
    } else if (ph == 6) {
      if (!wait(&g2, c.nmt * NDX)) return;
      for (int i = 0; i < c.nmt * NDX; ++i) check(dxp[i] == i / NDX, "dx read dXp not written", i, 0);
      dx[t] = 1;
    }
  }
  Launch launch(unsigned mask) {
    Launch L;
    L.nphases = 7;
    L.mask = mask;
    L.shape = [this](int ph, int& g, int& p, Claim& c) { return shape(ph, g, p, c); };
    L.body = [this](int ph, int t, const Claim& c) { body(ph, t, c); };
    return L;
  }
  bool complete() const {
    for (int e = 0; e < E; ++e)
      if (dw2[e] != 1 || dw13[e] != 1) return false;
    for (int t = 0; t < NC; ++t)
      if (dx[t] != 1) return false;
    return true;
  }
};

static void zero(std::vector<int>& q) {
  for (int& v : q) v = 0;
}

int main(int argc, char** argv) {
  if (argc != 4) {
    fprintf(stderr, "usage: %s <scenario> <workers> <seed>\n", argv[0]);
    return 2;
  }
  const std::string sc = argv[1];
  const int workers = atoi(argv[2]);
  const uint64_t seed = strtoull(argv[3], nullptr, 10);
  int32_t status = 0;
  if (sc.rfind("fwd", 0) == 0) {
    // fwd-drop: the held-back counter times out (a limit that the other
    // waits never reach); fwd-tiny: every wait has a tiny limit, so whichever
    // expires first aborts the call and the rest drain
    const bool drop = sc == "fwd-drop", tiny = sc == "fwd-tiny";
    FwdModel m(tiny ? 64 : drop ? 200000 : (1ll << 40), seed);
    if (drop) m.drop_tile = 0;
    if (sc == "fwd-single" || drop || tiny) {
      run_launch(m.qctr.data(), m.launch(0x7Fu), workers, seed);
    } else if (sc == "fwd-default") {
      // routing .. up projection | down projection | plain combine
      run_launch(m.qctr.data(), m.launch(0x1Fu), workers, seed);
      run_launch(m.qctr.data(), m.launch(0x20u), workers, seed + 1);
      m.plain_combine();
    } else {
      fprintf(stderr, "unknown scenario %s\n", sc.c_str());
      return 2;
    }
    status = m.status;
    if (tiny) {
      check(status == 0 || status == moe::proto::kErrTimeout, "tiny: unexpected status", status, 0);
    } else if (drop) {
      // the held-back counter must surface as a timeout, and no up
      // projection of that tile may have run
      check(status == moe::proto::kErrTimeout, "drop: status is not MOE_ERR_TIMEOUT", status, 0);
      check(!__atomic_load_n(&m.ran_up[0], __ATOMIC_RELAXED), "drop: an up projection of the held-back tile ran", 0, 0);
    } else {
      check(status == 0, "status set without a fault", status, 0);
      check(m.complete(), "outputs incomplete", 0, 0);
    }
  } else if (sc == "bwd-single" || sc == "bwd-default") {
    BwdModel m(1ll << 40, seed);
    if (sc == "bwd-single") {
      run_launch(m.qctr.data(), m.launch(0x7Fu), workers, seed);
    } else {
      const unsigned masks[6] = {0x03u, 0x04u, 0x08u, 0x10u, 0x20u, 0x40u};
      for (unsigned mk : masks) {
        zero(m.qctr);  // each launch has its own queues on the device too
        run_launch(m.qctr.data(), m.launch(mk), workers, seed + mk);
      }
    }
    status = m.status;
    check(status == 0, "status set without a fault", status, 0);
    check(m.complete(), "outputs incomplete", 0, 0);
  } else {
    fprintf(stderr, "unknown scenario %s\n", sc.c_str());
    return 2;
  }
  if (g_violations.load()) {
    fprintf(stderr, "%ld violations\n", g_violations.load());
    return 1;
  }
  printf("ok status=%d tasks=%ld\n", status, g_tasks.load());
  return 0;
}
