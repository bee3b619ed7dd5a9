// mxfp8.h -- MXFP8 (E4M3 elements, E8M0 scale per 32) kernels.
#pragma once

#include "plan.h"
#include "tasks_fwd.h"

namespace moe {

static int mxfp8_gather_perm(const bf16_t* x, const int* perm, uint8_t* xq, uint8_t* xs, int R, int d, int k,
                             hipStream_t st) {
  return MOE_ERR_UNSUPPORTED;
}
static int mxfp8_quantize_rows(const bf16_t* src, int64_t rows, int64_t K, uint8_t* codes, uint8_t* scales,
                               hipStream_t st) {
  return MOE_ERR_UNSUPPORTED;
}
static int mxfp8_forward(const Plan& p, const moe_desc* D, const Fwd& F, const moe_weights* w, hipStream_t st) {
  return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe
