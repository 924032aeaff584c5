// Backward kernels (placeholder until the gfx950 backward lands).
#pragma once

#include "../../include/blockattn.h"
#include "ba_common.h"

namespace ba {

static inline int bwd_impl(const ba_desc*, const ba_s2_desc*, const void*, const void*, const void*,
                           const void*, const void*, const float*, float*, float*, void*, void*,
                           int32_t, void*, int32_t, hipStream_t) {
  return BA_ERR_UNSUPPORTED;
}

}  // namespace ba
