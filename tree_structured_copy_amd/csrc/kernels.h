// Launchers for the HIP kernels (attn.hip, attn_rows.hip, attn_merge.hip, kv.hip).
#pragma once
#include <hip/hip_runtime_api.h>

#include "tkv_types.h"

namespace tkv {

// The fixed device workspace of tkv_attend_decode_noalloc (static_ws.hip): a
// file-scope device array of this many bytes on every device the library runs
// on.  static_workspace_init(device) looks its address up once per device
// (with that device made current); static_workspace(device) returns it, or
// nullptr before the init.  Nothing else may name the array.
constexpr size_t kStaticWorkspaceBytes = size_t(64) << 20;
int static_workspace_init(int device);
void* static_workspace(int device);

// Names of the kernels launched by this host thread since launch_log_reset(),
// "name<template arguments>" joined by ';' (a fixed buffer: nothing is
// allocated; names past its end are dropped).  The launchers below add theirs.
void launch_log_reset();
void launch_log_add(const char* name);
const char* launch_log();

// Partial attention over items [args.item0, args.item0 + n_items) whose groups
// need `tiles` row tiles of 16; grid = n_items * Hkv workgroups of 64 * waves
// threads (waves = 4 or 8).
// nt (decode only): the launch first writes these new tokens (write_new_tokens).
hipError_t launch_attn_partial(int dtype, int head_dim, int tiles, int waves, bool causal, const AttnArgs& args,
                               int32_t n_items, hipStream_t stream, const NewTokens* nt = nullptr);

// Partial attention for groups of 3..16 row tiles with K/V staged in LDS;
// grid = n_items * Hkv / (heads per workgroup) workgroups.  cus = the device's
// compute units (the ring depth depends on workgroups per CU).
hipError_t launch_attn_rows(int dtype, int head_dim, int tiles, bool causal, const AttnArgs& args, int32_t n_items,
                            hipStream_t stream, int cus, const NewTokens* nt = nullptr);

// Log-sum-exp merge of each query's partial records into out; one wave per
// (query, query head), four per workgroup.
hipError_t launch_attn_merge(int head_dim, const MergeArgs& args, hipStream_t stream);

// Scatter appended tokens into pool tiles; grid = nent x Hkv x layers.
hipError_t launch_append(int dtype, int head_dim, int32_t layers, const AppendArgs& args,
                         hipStream_t stream);

// Copy `bytes` (a multiple of 4; both pointers 16-byte aligned) from src, a
// device-visible pointer to pinned host memory, to dst in device memory;
// at most 1024 workgroups of 256.
hipError_t launch_plan_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);

// Write words[i].value at 32-bit word words[i].word of plan, for i < n, skipping
// words >= limit; grid = ceil(n / 256) workgroups of 256.
hipError_t launch_plan_patch(int32_t* plan, const PlanWord* words, int32_t n, uint32_t limit, hipStream_t stream);

// The same for args.n <= kPatchArgWords words held in the arguments; one
// workgroup of 512.
hipError_t launch_plan_patch_args(const PatchArgs& args, hipStream_t stream);

// A decode step's new tokens of one layer plus its plan's changed words, one
// launch; grid = (nent + (npatch > 0)) x Hkv.
hipError_t launch_decode_prep(int dtype, int head_dim, const DecodePrepArgs& args, hipStream_t stream);

// Copy a path's tiles back out in token order; grid = nent x Hkv.
hipError_t launch_gather(int dtype, int head_dim, const GatherArgs& args, hipStream_t stream);

}  // namespace tkv
