// Internal entry points shared by the C ABI translation units (api.cpp and
// noalloc.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/qat_attn.h"

namespace qat {

// The backward stages of qat_attn_bwd_stages on a caller-provided scratch
// buffer.  split_tail = false runs every dK/dV key block whole (no partial
// sums in the scratch).
int bwd_impl(const qat_attn_dims* dims, const void* q, const void* k, const void* v, const float* v_scale,
             const void* o_hp, const float* lse, const void* dout, float sm_scale, int causal,
             uint32_t quant_flags, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
             uint32_t stages, bool split_tail, void* stream);

// Scratch bytes of a whole backward with split_tail = false (0 for invalid dims).
size_t bwd_bytes_whole(const qat_attn_dims* dims, uint32_t quant_flags);

}  // namespace qat
