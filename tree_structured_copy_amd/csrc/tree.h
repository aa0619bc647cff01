// Host core: the copy-on-write node tree and its block allocator.
//
// Dendrite article (ainews.cool, "technical deep dive"): the cache is a tree; a
// shared prefix is stored once; forking at position t copies nothing below t and
// gives each branch new, empty leaves for later positions.  Here a node is a run
// of tokens that one branch appended after its parent was frozen; it owns the
// blocks holding them (every node starts at slot 0 of a fresh block).  A handle
// points at its tip node; its path is tip -> root.
//
// Invariants:
//  * node.refs = live children + handles whose tip is the node; a node with
//    refs == 0 is freed together with its blocks, so a node is live exactly
//    while some live handle's path contains it;
//  * a frozen node is never written again (sticky; set by fork);
//  * an unfrozen node has exactly one handle and no children.
#pragma once
#include <stdint.h>

#include <vector>

#include "tkv.h"

namespace tkv {

// Lowest-free-id block allocator over a two-level bitmap.
class BlockPool {
 public:
  void init(int32_t n);
  int32_t num_free() const { return free_; }
  int32_t size() const { return n_; }
  int32_t take();  // lowest free id, -1 if none
  void give(int32_t b);
  bool is_free(int32_t b) const { return (words_[b >> 6] >> (b & 63)) & 1; }

 private:
  std::vector<uint64_t> words_;    // bit set = block free
  std::vector<uint64_t> summary_;  // bit w set = words_[w] != 0
  int32_t n_ = 0;
  int32_t free_ = 0;
};

struct Node {
  int32_t parent = -1;
  int32_t refs = 0;
  int32_t nhandles = 0;
  int32_t depth = 0;
  int64_t base = 0;  // absolute position of the node's first token
  int64_t ntok = 0;
  bool frozen = false;
  bool live = false;
  std::vector<int32_t> blocks;

  int32_t tail_valid() const {
    return blocks.empty() ? 0 : static_cast<int32_t>(ntok - 16 * (int64_t)(blocks.size() - 1));
  }
  // Back to a fresh node, keeping the block list's memory for the next user
  // of this slot.
  void reset() {
    parent = -1;
    refs = nhandles = depth = 0;
    base = ntok = 0;
    frozen = live = false;
    blocks.clear();
  }
};

struct Handle {
  uint32_t gen = 0;
  int32_t tip = -1;
  bool live = false;
};

// Where the tokens of one append land: slots [first_slot, 16) of blocks[0]
// (first_slot == 0 means blocks[0] is fresh), then whole fresh blocks.
struct Placement {
  int32_t first_slot = 0;
  std::vector<int32_t> blocks;
};

class Tree {
 public:
  explicit Tree(int32_t num_blocks);

  int seq_new(tkv_seq* out);
  int fork(tkv_seq parent, int32_t n, tkv_seq* out);
  int release(tkv_seq s);
  int truncate(tkv_seq s, int64_t new_len);
  int append(tkv_seq s, int32_t ntok, Placement* pl);
  // Fresh blocks append(s, ntok) would take (validates s and ntok like it).
  int append_need(tkv_seq s, int32_t ntok, int64_t* blocks) const;
  // Undo the metadata of the latest successful append (used when its device
  // part could not be launched).  Only valid immediately after that append.
  void undo_append(tkv_seq s, int32_t ntok, const Placement& pl, bool made_node);

  int seq_len(tkv_seq s, int64_t* len) const;
  // Block and slot of s's last token when it lies in s's own tip node (never
  // forked, so no other handle shares it); TKV_E_EMPTY if s has no token,
  // TKV_E_SHARED if its last token is shared with other branches.
  int own_last_token(tkv_seq s, int32_t* block, int32_t* slot) const;
  int block_table(tkv_seq s, int32_t* ids, int32_t* valid, int32_t cap, int32_t* n) const;
  int block_refcounts(int32_t* rc) const;
  int block_refcount(int32_t b, int32_t* rc) const;
  int num_free() const { return pool_.num_free(); }
  int32_t num_blocks() const { return pool_.size(); }
  // Slot of a handle (valid after resolve() succeeded on it), and the number
  // of slots, for per-handle marks kept outside the tree.
  static uint32_t slot_of(tkv_seq s) { return static_cast<uint32_t>(s & 0xffffffffu); }
  size_t handle_slots() const { return handles_.size(); }

  // For the planner.
  int resolve(tkv_seq s, int32_t* tip) const;
  const Node& node(int32_t id) const { return nodes_[id]; }
  int32_t node_capacity() const { return static_cast<int32_t>(nodes_.size()); }
  // epoch: bumped by every change.  shape_epoch: bumped by every change except
  // an append that fits in its tip node's last block (it then changes only
  // that block's valid count and the handle's length).
  uint64_t epoch() const { return epoch_; }
  uint64_t shape_epoch() const { return shape_epoch_; }
  bool last_append_made_node() const { return last_made_node_; }

  tkv_counters counters{};

 private:
  int32_t new_node();
  void free_node(int32_t id);
  int32_t new_handle(int32_t tip, tkv_seq* out);

  std::vector<Node> nodes_;
  std::vector<int32_t> free_nodes_;
  std::vector<Handle> handles_;
  std::vector<int32_t> free_handles_;
  std::vector<int32_t> block_owner_;  // node owning each used block
  BlockPool pool_;
  uint64_t epoch_ = 1;
  uint64_t shape_epoch_ = 1;
  bool last_made_node_ = false;
};

}  // namespace tkv
