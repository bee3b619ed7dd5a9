// slots.h -- where the buffers exchanged inside one persistent launch put
// each producer's bytes, written once for the kernels and for a host check
// (tests/exchange_lines.cpp) that no 128-byte line holds bytes of two
// producers.  The consumers of these buffers invalidate no cache (common.h),
// so a line shared by two producers could be read by one consumer before
// the other producer wrote its part and then served stale from that
// consumer's L1 or L2.
//
// The includer defines MOE_PROTO_FN (the function qualifiers).
#pragma once

#include <stddef.h>
#include <stdint.h>

#ifndef MOE_PROTO_FN
#error "define MOE_PROTO_FN (the function qualifiers) before including slots.h"
#endif

namespace moe {
namespace slots {

constexpr int kLine = 128;  // bytes per cache line (L1 and L2)

// Element index of row i of row tile `tile` in an array with one slot of
// BM rows per row tile (rows of `per_row` elements).  A slot holds BM *
// per_row elements; with BM a multiple of 32 rows of 4-byte elements, or
// of BM * per_row bytes a multiple of 128, every slot starts on a line.
MOE_PROTO_FN size_t tile_slot(int tile, int i, int BM, size_t per_row) {
  return ((size_t)tile * BM + i) * per_row;
}

// Floats per slice of the router's partial logits: T E rounded up to 32
// (128 bytes), so that each slice starts on a line (slices are written by
// different tasks and the top-k tasks read all of them).
MOE_PROTO_FN size_t router_slice_stride(int T, int E) {
  return (((size_t)T * E) + 31) & ~(size_t)31;
}

}  // namespace slots
}  // namespace moe
