// Calls between the library's own host files, outside the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "k3moe.h"

namespace k3 {

// The router logits alone (no top-k) of handle h for x [T][d] bf16 into
// logits [T][E] fp32 (device), on stream st. The router bias is added unless
// the handle ranks with a selection-only bias. Returns a K3MOE_* status;
// arguments as k3moe_route, with logits required.
int route_logits(k3moe* h, const void* x, int32_t T, float* logits, hipStream_t st);

}  // namespace k3
