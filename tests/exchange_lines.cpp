// exchange_lines.cpp -- host check that no 128-byte line of a buffer
// exchanged inside one persistent launch holds bytes of two producers that
// a consumer may wait for separately.  Built and run by
// tests/test_protocol_model.py.
//
// Test infrastructure.  The consumers of these buffers poll a counter and
// invalidate no cache (csrc/common.h), so a consumer that reads a line
// shared with another producer's still-unwritten bytes would later serve
// those bytes stale from its L1 or L2.  The producers are grouped by the
// counter their consumers wait on: a row tile (its gather; its up-projection
// column tiles, all of which a down-projection tile waits for), a 64-token
// block of the router slices.  The slot addresses come from csrc/slots.h,
// the same functions the kernels use.
//
// Layouts checked over random expert loads (empty experts, ragged tails,
// one expert holding every token): the tile-slotted source index and MXFP8
// H scales, the router slices, the gathered rows (d * 2 bytes), H (I * 2),
// H codes (I); and, to show that the check can fail, the source index laid
// out by row (4 bytes per routed row), which must share lines for some
// loads.
//
// usage: exchange_lines <iterations> <seed>; prints "ok <n>" or the first
// shared line and exits 1
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <vector>

#define MOE_PROTO_FN inline
#include "../mixture_experts_layer_layout_amd/csrc/slots.h"

using moe::slots::kLine;

struct Range {
  long long group, lo, hi;  // bytes [lo, hi) written by producer group `group`
};

// The first line touched by two groups, or -1.  Ranges sorted by start:
// a line is shared exactly when a range starts on or before the last line
// reached so far by a range of another group.
static long long shared_line(std::vector<Range> rs) {
  std::sort(rs.begin(), rs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  long long last = -1, last_group = -1;
  for (const Range& r : rs) {
    if (r.hi <= r.lo) continue;
    const long long first = r.lo / kLine, end = (r.hi - 1) / kLine;
    if (first <= last && r.group != last_group) return first;
    if (end > last) {
      last = end;
      last_group = r.group;
    }
  }
  return -1;
}

struct TileRow {
  int e, r0, n;
};

int main(int argc, char** argv) {
  const int iters = argc > 1 ? atoi(argv[1]) : 200;
  std::mt19937_64 rng(argc > 2 ? strtoull(argv[2], nullptr, 10) : 1);
  int old_layout_shared = 0;
  for (int it = 0; it < iters; ++it) {
    const int Es[] = {1, 8, 32, 256};
    const int E = Es[rng() % 4];
    int k = 1 + (int)(rng() % 8);
    if (k > E) k = E;
    const int T = 1 + (int)(rng() % 3000);
    const int BM = (rng() % 2) ? 128 : 256;
    const int Is[] = {128, 256, 2048, 14336};
    const int I = Is[rng() % 4];
    const int ds[] = {256, 4096, 7168};
    const int d = ds[rng() % 3];
    // expert loads: each token picks k distinct experts -- uniformly, the
    // first k experts (one-hot routing), or skewed (a random order of the
    // experts, taken with probability falling along it)
    std::vector<int> cnt(E, 0);
    const int mode = (int)(rng() % 3);
    for (int t = 0; t < T; ++t) {
      std::vector<int> ids(E);
      for (int e = 0; e < E; ++e) ids[e] = e;
      for (int j = 0; j < k; ++j) {
        int pick = j;  // mode 2: experts 0 .. k-1
        if (mode == 0) pick = j + (int)(rng() % (E - j));
        if (mode == 1) pick = j + (int)((rng() % (E - j)) * (rng() % (E - j)) / (E - j));
        std::swap(ids[j], ids[pick]);
        ++cnt[ids[j]];
      }
    }
    // row tiles as the layout scan lists them
    std::vector<TileRow> tiles;
    int off = 0;
    for (int e = 0; e < E; ++e) {
      for (int mt = 0; mt * BM < cnt[e]; ++mt) tiles.push_back({e, off + mt * BM, std::min(BM, cnt[e] - mt * BM)});
      off += cnt[e];
    }
    std::vector<Range> tsrc, hs, xp, h, hq, src_by_row;
    for (size_t ti = 0; ti < tiles.size(); ++ti) {
      const TileRow& tr = tiles[ti];
      const long long g = (long long)ti;
      tsrc.push_back({g, (long long)moe::slots::tile_slot((int)ti, 0, BM, 1) * 4,
                      (long long)moe::slots::tile_slot((int)ti, tr.n, BM, 1) * 4});
      // MXFP8 tiles have 128 rows; the up-projection column tiles of a row
      // tile write the I/32 scale bytes of each of its rows (one group: the
      // down projection waits for all of them)
      if (BM == 128)
        for (int row = 0; row < tr.n; ++row) {
          const long long b = (long long)moe::slots::tile_slot((int)ti, row, BM, I / 32);
          hs.push_back({g, b, b + I / 32});
        }
      xp.push_back({g, (long long)tr.r0 * d * 2, (long long)(tr.r0 + tr.n) * d * 2});
      h.push_back({g, (long long)tr.r0 * I * 2, (long long)(tr.r0 + tr.n) * I * 2});
      hq.push_back({g, (long long)tr.r0 * I, (long long)(tr.r0 + tr.n) * I});
      src_by_row.push_back({g, (long long)tr.r0 * 4, (long long)(tr.r0 + tr.n) * 4});
    }
    // router slices: task (block b, slice s) writes rows 64b .. of slice s;
    // the top-k tasks of block b wait for all S slices of b
    std::vector<Range> lpart;
    const int S = 4, nb = (T + 63) / 64;
    const size_t stride = moe::slots::router_slice_stride(T, E);
    for (int s = 0; s < S; ++s)
      for (int b = 0; b < nb; ++b) {
        const int t1 = std::min(64 * b + 64, T);
        lpart.push_back({b, (long long)(s * stride + (size_t)64 * b * E) * 4, (long long)(s * stride + (size_t)t1 * E) * 4});
      }
    struct {
      const char* name;
      const std::vector<Range>* r;
    } bufs[] = {{"tile-slotted source index", &tsrc}, {"tile-slotted H scales", &hs}, {"router slices", &lpart},
                {"gathered rows", &xp}, {"H rows", &h}, {"H code rows", &hq}};
    for (auto& b : bufs) {
      const long long l = shared_line(*b.r);
      if (l >= 0) {
        printf("FAIL %s: line %lld shared (T=%d E=%d k=%d BM=%d I=%d d=%d)\n", b.name, l, T, E, k, BM, I, d);
        return 1;
      }
    }
    if (shared_line(src_by_row) >= 0) ++old_layout_shared;
  }
  if (old_layout_shared == 0) {
    printf("FAIL the row-indexed source index never shared a line: the check cannot fail\n");
    return 1;
  }
  printf("ok %d (row-indexed layout shared lines in %d)\n", iters, old_layout_shared);
  return 0;
}
