// Library-internal entry points of the host layer (attn_api.cpp) shared with
// other sources of the library; not part of the C ABI.
#pragma once

#include "../../include/attn.h"

namespace attn {

// Every check attn_bwd makes except those on the workspace (its pointer, size,
// alignment and aliasing), with no HIP call: ATTN_OK means attn_bwd would
// accept these arguments together with any valid, non-aliasing workspace.
attn_status bwd_validate_without_workspace(const attn_params* p, const void* q, const void* k,
                                           const void* v, const void* o, const float* lse,
                                           const void* d_o, void* dq, void* dk, void* dv);

}  // namespace attn
