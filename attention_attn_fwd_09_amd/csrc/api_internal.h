// Internal entry shared by the backward entry points of the C ABI (no device code here).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "attn.h"

namespace attn {

// Supplies the workspace of a call once every other host-side check has passed: given the bytes
// the call needs, sets *workspace and *bytes, or returns the status that rejects the call.
typedef attn_status (*WorkspaceProvider)(size_t need, void** workspace, size_t* bytes);

// attn_bwd_ex with an optional workspace provider (null: the caller's workspace arguments are used).
attn_status bwd_call(const attn_problem* problem, const void* Q, const void* K, const void* V, const void* O,
                     const void* dO, const float* LSE, const attn_mask* mask, float scale, void* dQ, void* dK,
                     void* dV, void* workspace, size_t workspace_bytes, int32_t flags, void* stream,
                     WorkspaceProvider provide);

}  // namespace attn
