// Internal entries shared by the entry points of the C ABI (no device code here).
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

// attn_fwd_ex (plan_bwd false) and attn_fwd_with_bwd_plan (plan_bwd true: one planner launch also
// writes the backward's two lists into bwd_workspace).
attn_status fwd_call(const attn_problem* problem, const void* Q, const void* K, const void* V,
                     const attn_mask* mask, float scale, void* O, float* LSE, void* workspace,
                     size_t workspace_bytes, int32_t kv_splits, void* bwd_workspace, size_t bwd_workspace_bytes,
                     bool plan_bwd, void* stream);

}  // namespace attn
