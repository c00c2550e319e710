// Internal entry of the host side shared by moe_forward (moe_api.cpp) and
// moe_forward_noalloc (noalloc.hip).
#pragma once

#include "moe.h"

namespace moe {

// moe_forward: every argument check, then the launches, with the workspace
// ws of ws_bytes bytes (MOE_ERR_WORKSPACE when it is NULL or too small; the
// other checks run first).
int forward_impl(const moe_shape *s, const void *x, int act, const void *wg, const float *bias,
                 const moe_expert_weights *w, void *y, int out, int32_t *topk_idx,
                 float *topk_w, void *ws, size_t ws_bytes, void *stream);

}  // namespace moe
