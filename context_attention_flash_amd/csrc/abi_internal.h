// Host entry points shared between the C ABI sources (not part of the ABI).
#pragma once

#include <cstddef>
#include <cstdint>

#include "ring_attn.h"

namespace ra {

// ring_attn_bwd with an explicit workspace; with build_plan = false a shape
// whose plan is not cached fails with RA_E_NO_PLAN instead of allocating one.
int bwd_impl(const ring_attn_desc* desc, const void* dout, const void* q, const void* k,
             const void* v, const void* out, const float* lse, const int32_t* cu, float* dq,
             float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream,
             bool build_plan);

// The minimum backward workspace of a descriptor (negative RA_E_* if invalid).
int64_t bwd_need_bytes(const ring_attn_desc* desc);

}  // namespace ra
