// dispatch.hpp -- per-shape GEMM configuration choice (internal, host only).
#pragma once

#include <stdint.h>

#include "../../include/fp8blk.h"

namespace fp8blk {

// Fills *out with the configuration for (M, N, K).  Arguments are validated
// by the caller.
void select_config(int64_t M, int64_t N, int64_t K, uint32_t flags, fp8blk_gemm_config* out);

}  // namespace fp8blk
