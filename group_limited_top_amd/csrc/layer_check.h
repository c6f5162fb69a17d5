// layer_check.h -- host-side argument checks of the layer forward, shared by
// its entry points (internal).
#pragma once

#include "moe.h"

namespace moe {

// moe_workspace_size's validation of a desc: MOE_OK, MOE_ERR_INVALID or
// MOE_ERR_UNSUPPORTED.
int validate_desc(const moe_desc_t* desc);

// Every check moe_layer_forward makes before it launches anything (the desc,
// required pointers, aliasing, weights, workspace size and alignment);
// launches nothing.
int layer_forward_check(const moe_desc_t* desc, const void* x, const moe_weights_t* weights,
                        void* y, int32_t* topk_idx_out, float* topk_w_out, float* logits_out,
                        int32_t* counts_out, int64_t* tracking, void* ws, size_t ws_bytes);

}  // namespace moe
