// Host planner: turns a batch of handles (and query counts) into the work list
// the attention kernels run.
//
// The article (ainews.cool, "technical deep dive") has attention walk the tree,
// reading K/V from the shared ancestor path and the branch's leaf path.  Reading
// that literally per query would fetch a shared prefix once per branch and per
// query head.  The planner instead:
//   1. collects the union of the batch's paths as a tree of nodes;
//   2. cuts it into groups of queries (at most kMaxRows rows = queries x heads per
//      KV head) that lie close together in the tree, never mixing independent
//      trees, so that one pass over a group's blocks serves all its rows;
//   3. lists each group's blocks once (root first, in position order), with a
//      mask of the group's queries that can see each block;
//   4. splits long lists into work items (split-K), one workgroup per item and
//      KV head, and records where each query's partial results go.
#pragma once
#include <stdint.h>

#include <memory>
#include <new>
#include <utility>
#include <vector>

#include "tkv_types.h"
#include "tree.h"

namespace tkv {

// Cost of a block's memory time in the planner's chunking of LDS-staged
// groups, in units of one more row tile's work on it.  Measured on the search
// tree (2048-token root, 256 leaves; 8-tile groups cut into 6 chunks each):
// 56.0 us per call with equal-length chunks; 69.6, 58.0, 52.7, 51.6, 51.4,
// 52.2 and 54.9 us at 2, 4, 8, 16, 24, 32 and 64.
constexpr int64_t kPlanBlockCost = 20;

// An allocator whose resize() leaves new elements uninitialised: the planner
// writes every field of each block entry it appends, and value-initialising
// them first was a second pass over the block list (half of its time on a
// 49 152-block plan).
template <class T>
struct NoInitAlloc : std::allocator<T> {
  template <class U>
  struct rebind {
    using other = NoInitAlloc<U>;
  };
  NoInitAlloc() = default;
  template <class U>
  NoInitAlloc(const NoInitAlloc<U>&) noexcept {}
  template <class U>
  void construct(U* p) noexcept {
    ::new (static_cast<void*>(p)) U;
  }
  template <class U, class... A>
  void construct(U* p, A&&... a) {
    ::new (static_cast<void*>(p)) U(std::forward<A>(a)...);
  }
};

struct PlanOptions {
  int32_t target_wgs = 256;
  int32_t min_chunk = 32;
  // Groups of at most 128 rows (8 row tiles) by default: a search tree's
  // leaves then run in one launch of the 8-tile shape, two workgroups per CU,
  // each group reading its private nodes with the shared ones; this measured
  // faster than 16-tile groups with their narrow nodes moved to one-tile
  // subgroups (the cascade, kept as an option) on every search-tree shape
  // tried, and the same on the fork and verify workloads.
  int32_t max_rows = 128;
  int32_t cascade = 0;  // split narrow blocks of large groups into one-tile subgroups
  // 1: a CU holds two workgroups of the 4- and 8-tile LDS-staged shapes, and
  // the 6-tile shape's workgroups hold two KV heads (or two fit a CU), so
  // one round of those classes is twice target_wgs / Hkv items (bf16, or
  // d <= 64); 0: one workgroup of one KV head per CU (fp32 at d = 128)
  int32_t two_per_cu = 1;
};

struct Plan {
  // Items sorted by kernel class (kernel_class() of their group's row tiles);
  // class c = items [bucket_begin[c], bucket_begin[c + 1]).
  std::vector<DevItem> items;
  int32_t bucket_begin[kKernelClasses + 1] = {0, 0, 0, 0, 0, 0, 0};
  int32_t bucket_tiles[kKernelClasses] = {1, 2, 4, 6, 8, 16};
  int32_t bucket_max_blocks[kKernelClasses] = {0, 0, 0, 0, 0, 0};  // longest item of each class
  int64_t bucket_blocks[kKernelClasses] = {0, 0, 0, 0, 0, 0};      // blocks of all items of each class
  std::vector<DevGroup> groups;
  std::vector<int32_t> gq;
  std::vector<int32_t> gqpos;
  std::vector<DevBlock, NoInitAlloc<DevBlock>> blocks;  // each entry written in full by the planner
  std::vector<DevPart> parts;
  std::vector<DevMerge> merge;
  int32_t nqueries = 0;
  int64_t partial_slots = 0;  // records of (m, l, acc[D])
  bool any_merge = false;
  bool causal = false;
  // statistics
  int32_t unique_blocks = 0;
  int64_t unique_tokens = 0;
  // What an append inside a tip node's last block can change, for patch_plan:
  // the last block entry of every listing of an unfrozen node; each query's
  // tip node and distance from the end (its position = length - back); the
  // distinct unfrozen nodes read, and the tokens of all other nodes read.
  std::vector<int32_t> tail_entry, tail_node;
  std::vector<int32_t> gq_node, gq_back;
  std::vector<int32_t> open_nodes;
  int64_t closed_tokens = 0;

  // serialised layout (byte offsets into one device buffer)
  size_t off_items = 0, off_gq = 0, off_gqpos = 0, off_blocks = 0,
         off_parts = 0, off_merge = 0, bytes = 0;
  void layout();
  void serialise(void* dst) const;
  // Empty every list (keeping its memory) and zero every count.
  void reset();
};

struct PlanQuery {
  int32_t handle;  // batch index
  int32_t global;  // global query index (row of q / out)
  int32_t pos;     // absolute position
};

struct PlanItemTmp {
  DevItem it;
  int32_t tiles, root, chunk;
};

// Working memory of build_plan, kept between calls so that rebuilding a plan
// of a size seen before allocates nothing.  `loc` is all -1 between calls.
struct PlanScratch {
  std::vector<int32_t> loc;  // tree node -> local node
  std::vector<int32_t> tip, qn, qbase;
  std::vector<int64_t> len;
  // local nodes: tree node, parent, handles (hlist[hbeg[k] .. hbeg[k + 1])),
  // children (child[cbeg[k] .. cbeg[k + 1]), by tree node), DFS preorder
  std::vector<int32_t> lnode, lparent, hbeg, hlist, cbeg, child, cursor, roots, pre, by_pre, st, sub;
  std::vector<int64_t> qcount;
  // query runs: units of one tree (ub), groups (gbeg, gsize, groot)
  std::vector<PlanQuery> uq;
  std::vector<int32_t> ub, gbeg, gsize, groot;
  std::vector<uint64_t> mask;
  std::vector<int32_t> touched;
  // cascade: each touched node's one-tile subgroup (or -1); the narrow nodes
  // by subgroup (sorder[sbeg[t] .. sbeg[t + 1]), indices into touched)
  std::vector<int32_t> nar, sbeg, sorder;
  std::vector<uint8_t> emitted;
  std::vector<int32_t> go_begin, go_count, go_root;
  std::vector<uint8_t> go_partials;
  std::vector<int64_t> go_cost;   // per group: chunking cost of its blocks (see kPlanBlockCost)
  std::vector<uint64_t> go_mask;  // per group: the queries that see any of its blocks
  std::vector<uint8_t> qm_n;
  std::vector<int32_t> qm_g, qm_j;
  std::vector<int8_t> gclass;
  std::vector<PlanItemTmp> tmp;
  std::vector<int32_t> ibeg, ilist;
  std::vector<uint32_t> tile_of_byte;
  int32_t tile_of_byte_qpk = 0;  // the query heads per KV head tile_of_byte was made for
  std::vector<int32_t> cut;
  std::vector<int64_t> gcost;  // per group: blocks (register classes) or chunking cost (LDS-staged)
  std::vector<int32_t> gchunks;
  std::vector<double> gfrac;
};

// Which kernel runs a group of `tiles` row tiles of 16: 0, 1 = attn.hip with 1
// or 2 tiles in every wave's registers (waves split the blocks); 2..5 =
// attn_rows.hip with the K/V staged in LDS and up to 4, 6, 8, 16 tiles spread
// over the waves.
inline int kernel_class(int tiles) {
  return tiles <= 1 ? 0 : tiles == 2 ? 1 : tiles <= 4 ? 2 : tiles <= 6 ? 3 : tiles <= 8 ? 4 : 5;
}

// Build the plan for a decode (nq == nullptr) or verify call.  Validates the
// handles (TKV_E_BADSEQ), query counts (TKV_E_RANGE) and emptiness (TKV_E_EMPTY).
// Bring a plan built from `tree` up to date after appends that each fitted in
// their tip node's last block (the tree's shape_epoch unchanged since the
// build): valid counts of those blocks, query positions and their minima, and
// the statistics.  The result equals a fresh build_plan.  Every 32-bit word of
// the serialised plan that changed is appended to `changed` (if given).
void patch_plan(const Tree& tree, Plan* plan, std::vector<PlanWord>* changed);

// `scratch` (optional) is working memory reused across calls.
int build_plan(const Tree& tree, const tkv_seq* seqs, const int32_t* nq, int32_t nseq,
               int32_t q_per_kv, int32_t num_kv_heads, const PlanOptions& opt, Plan* out,
               PlanScratch* scratch = nullptr);

}  // namespace tkv
