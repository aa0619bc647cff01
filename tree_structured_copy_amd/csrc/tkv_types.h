// Plain structs shared by the host planner and the HIP kernels.
#pragma once
#include <stdint.h>

namespace tkv {

constexpr int kBlock = 16;          // token slots per block
constexpr int kMaxRows = 256;       // rows (queries x heads-per-kv-head) per group
constexpr int kMaxGroupQueries = 64; // one bit per query in a block's visibility mask
constexpr int kKernelClasses = 6;   // A1, A2 (attn.hip), B4, B6, B8, B16 (attn_rows.hip)
constexpr int kRowsMaxItemBlocks = 1024;  // longest block list of one attn_rows.hip work item (16 KiB of LDS)
constexpr int kMaxPoolBlocks = 1 << 27;   // block ids fit 27 bits (attn_rows.hip packs the valid count beside them)
constexpr int kAppendMaxBlocks = 128;   // blocks per decode-step preparation launch
constexpr int kAppendWideBlocks = 240;  // blocks per plain append launch
constexpr int kGatherMaxBlocks = 64;

// A query group: up to kMaxRows rows that share one pass over the union of
// their paths.  Its queries are gq[q_begin .. q_begin + nq); min_pos is the
// smallest position limit among them (keys at or below it are visible to all).
// (Host side: every work item carries its group's fields.)
struct DevGroup {
  int32_t q_begin;
  int32_t nq;
  int32_t min_pos;
  int32_t pad1;
};

// One work item: a contiguous run of a group's block list, processed by one
// workgroup per KV head, with its group's query range and position limit (so
// a workgroup needs no group record before it can load its queries).
// part_base < 0: the item covers its group's whole list and writes normalised
// outputs directly; otherwise it writes fp32 partial records (m, l, acc) at
// slots part_base + j * Hq + h for the queries j in qmask.
// tails: the item's blocks that end an unfrozen node (a branch's tip block,
// where a decode step's new token goes) are the plan's tail blocks
// [tails & 0xffff, + (tails >> 16)) in block-list order; 0 when there are
// none or the indices do not fit 16 bits.
// qmask: the group queries that see at least one of the item's blocks; an
// item with partial records writes records for these queries only (the
// merge lists no record of an item for a query that sees none of its blocks).
struct DevItem {
  int32_t group;
  int32_t blk_begin;
  int32_t blk_count;
  int32_t part_base;
  int32_t q_begin;
  int32_t nq;
  int32_t min_pos;
  int32_t tails;
  uint64_t qmask;
  int32_t pad0;
  int32_t pad1;
};

// One block on a group's path list.  mask bit j = group query j can see the
// block; pos = absolute position of slot 0; valid = slots in use.
struct DevBlock {
  int32_t id;
  int32_t pos;
  int32_t valid;
  int32_t pad;
  uint64_t mask;
};

// One partial record of a query: the work item that wrote it put query head h
// at slot slot0 + h (slot0 = the item's part_base + j * Hq, j = the query's
// index in the item's group).  A query's records are parts[p_begin ..
// p_begin + p_count) of its DevMerge; p_count == 0: its output was written
// directly.
struct DevPart {
  int32_t slot0;
  int32_t item;  // for checks and statistics; the merge does not read it
};
struct DevMerge {
  int32_t p_begin;
  int32_t p_count;
};

// One 32-bit word of a serialised plan to overwrite in place (the device copy
// of a plan brought up to date after appends inside tip blocks).
struct PlanWord {
  uint32_t word;  // byte offset / 4
  int32_t value;
};

// Changed words passed to the patch kernel as its arguments (no copy of the
// list beforehand): up to kPatchArgWords per launch, within the 4 KiB
// kernel-argument limit.
constexpr int kPatchArgWords = 480;
struct PatchArgs {
  int32_t* plan;
  int32_t n;
  uint32_t limit;
  PlanWord w[kPatchArgWords];
};

struct AttnArgs {
  const void* kpool;  // layer base
  const void* vpool;
  const void* q;
  float* out;
  const DevItem* items;
  const int32_t* gq;     // global query index per group slot
  const int32_t* gqpos;  // absolute position limit per group slot
  const DevBlock* blocks;
  float* part_acc;       // [slots][D] unnormalised sums of exp2((s - m) * scale_log2) V
  float* part_ml;        // [slots][2]: running max m (raw score units) and sum l
  int32_t hq;
  int32_t hkv;
  int32_t gsize;         // Hq / Hkv
  int32_t item0;         // first item of this launch
  float scale_log2;      // log2(e) / sqrt(D)
  int32_t max_blocks;    // the longest block list among this launch's items
};

// The new tokens of one branch in a decode step, written by the attention
// launch itself (tkv_attend_decode_new_token(s) in one launch): plan block
// entry `entry` (an index into the plan's block list) is the tokens' block
// `blk`, which takes `n` tokens at slots slot .. slot + n - 1 from rows
// src .. src + n - 1 of the call's K/V arrays.  The launch's list is indexed by
// the plan's tail blocks (DevItem::tails); entry = -1 where a tail block takes
// no token in this call.
struct NewTok {
  int32_t entry;
  int32_t blk;
  int16_t slot;
  int16_t n;
  int32_t src;
};
// A block id of a plan's device copy that the attention launch rewrites
// before reading it: a cached plan's device copy reused for another batch of
// the same shape (a search step's new leaves under a node at the depth of an
// earlier one), whose only differences are the block ids.
struct IdPatch {
  int32_t entry;  // index into the plan's block list
  int32_t id;
};
// Up to this many new tokens and id patches travel in an attention launch's
// arguments (with AttnArgs, within the 4 KiB kernel-argument limit).
constexpr int kFusedMaxTokens = 192;
constexpr int kMaxIdPatches = 64;
struct NewTokens {
  static constexpr bool kActive = true;
  const void* k;     // [rows][Hkv][D] of the call's layer
  const void* v;
  void* kpool;       // the layer's base
  void* vpool;
  DevBlock* blocks;  // the plan's block list: the tokens' valid counts and patched ids are written here
  int32_t n;         // tail blocks listed (tok[0 .. n)), 0 = no tokens
  int32_t nid;       // id patches (ids[0 .. nid)), 0 = none
  int32_t multi;     // 1: some record holds several tokens (each workgroup writes its records together first)
  NewTok tok[kFusedMaxTokens];
  IdPatch ids[kMaxIdPatches];
};
// A launch that writes no token (an empty argument).
struct NoNewTokens {
  static constexpr bool kActive = false;
};

struct MergeArgs {
  const DevPart* parts;
  const DevMerge* merge;
  const float* part_acc;
  const float* part_ml;
  float* out;
  int32_t hq;
  int32_t nq;
  float scale_log2;    // partial maxima are raw scores: weights are exp2((m - M) * scale_log2)
  int32_t pad;
};

// One block an append writes: slots [slot, slot + cnt) of block blk take
// source token rows [src, src + cnt); slot == 0 means the block is fresh (its
// other slots are zeroed).
struct AppendEntry {
  int32_t blk;
  int32_t slot;
  int32_t src;
  int32_t cnt;
};

// An append launch: the source arrays, the pools and up to N blocks to write
// (in the kernel's arguments).
template <int N>
struct AppendArgsN {
  const void* src_k;   // [L][ntok][Hkv][D]
  const void* src_v;
  void* kpool;         // pool base (layer 0)
  void* vpool;
  int64_t layer_stride;  // elements per layer of a pool
  int32_t ntok;        // token rows in the source arrays
  int32_t hkv;
  int32_t nent;        // blocks in this launch
  int32_t pad[3];
  AppendEntry ent[N];
};
// a plain append launch: as many blocks as the 4 KiB argument limit allows
using AppendArgs = AppendArgsN<kAppendWideBlocks>;
// the blocks part of a decode step's preparation launch, which also carries
// the plan's changed words
using PrepAppendArgs = AppendArgsN<kAppendMaxBlocks>;

// The preparation launch of a decode step that writes its new tokens
// (tkv_attend_decode_new_token): the tokens of one layer (app: a one-layer
// source, pools at that layer's base) and up to kPrepPatchWords changed words
// of the call's plan, all in the kernel's arguments (within the 4 KiB limit).
constexpr int kPrepPatchWords = 240;
struct DecodePrepArgs {
  PrepAppendArgs app;
  int32_t* plan;
  int32_t pad0;
  int32_t npatch;
  uint32_t limit;
  int32_t pad;
  PlanWord patch[kPrepPatchWords];
};

struct GatherArgs {
  const void* kpool;   // layer base
  const void* vpool;
  void* k_out;         // [len][Hkv][D]
  void* v_out;
  int32_t hkv;
  int32_t nent;
  int32_t blk[kGatherMaxBlocks];
  int32_t valid[kGatherMaxBlocks];
  int32_t pos[kGatherMaxBlocks];
};

}  // namespace tkv
