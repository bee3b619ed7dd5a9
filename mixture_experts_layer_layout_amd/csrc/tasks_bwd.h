// tasks_bwd.h -- the backward of the expert path as tasks.
#pragma once

#include "plan.h"
#include "tasks_fwd.h"

namespace moe {

static int backward_impl(const Plan& p, const moe_desc* D, const void* dy, const void* x, const moe_weights* w,
                         const moe_saved* sv, void* dx, void* dw1, void* dw3, void* dw2, float* dgate, void* ws,
                         hipStream_t st) {
  return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe
