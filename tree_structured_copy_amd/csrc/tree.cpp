#include "tree.h"

#include <algorithm>
#include <new>

namespace tkv {

namespace {

// Room for `more` further elements, growing geometrically: an exact reserve
// reallocates (and moves every element) on each call, which would make fork
// O(handles) and node creation O(nodes).
template <class V>
void make_room(V& v, size_t more) {
  const size_t need = v.size() + more;
  if (v.capacity() < need) v.reserve(std::max(need, 2 * v.capacity()));
}

}  // namespace

// ---------------------------------------------------------------- BlockPool

void BlockPool::init(int32_t n) {
  n_ = n;
  free_ = n;
  words_.assign((n + 63) / 64, 0);
  summary_.assign((words_.size() + 63) / 64, 0);
  for (int32_t b = 0; b < n; ++b) words_[b >> 6] |= 1ull << (b & 63);
  for (size_t w = 0; w < words_.size(); ++w)
    if (words_[w]) summary_[w >> 6] |= 1ull << (w & 63);
}

int32_t BlockPool::take() {
  for (size_t s = 0; s < summary_.size(); ++s) {
    if (!summary_[s]) continue;
    const size_t w = s * 64 + __builtin_ctzll(summary_[s]);
    const int bit = __builtin_ctzll(words_[w]);
    words_[w] &= ~(1ull << bit);
    if (!words_[w]) summary_[s] &= ~(1ull << (w & 63));
    --free_;
    return static_cast<int32_t>(w * 64 + bit);
  }
  return -1;
}

void BlockPool::give(int32_t b) {
  const size_t w = static_cast<size_t>(b) >> 6;
  words_[w] |= 1ull << (b & 63);
  summary_[w >> 6] |= 1ull << (w & 63);
  ++free_;
}

// ---------------------------------------------------------------- Tree

Tree::Tree(int32_t num_blocks) {
  pool_.init(num_blocks);
  block_owner_.assign(num_blocks, -1);
}

int32_t Tree::new_node() {
  int32_t id;
  if (!free_nodes_.empty()) {
    id = free_nodes_.back();
    free_nodes_.pop_back();
    nodes_[id].reset();
  } else {
    id = static_cast<int32_t>(nodes_.size());
    nodes_.emplace_back();
  }
  nodes_[id].live = true;
  ++counters.nodes_created;
  return id;
}

void Tree::free_node(int32_t id) {
  Node& n = nodes_[id];
  for (int32_t b : n.blocks) {
    pool_.give(b);
    block_owner_[b] = -1;
    ++counters.blocks_freed;
  }
  n.reset();
  free_nodes_.push_back(id);
  ++counters.nodes_freed;
}

int32_t Tree::new_handle(int32_t tip, tkv_seq* out) {
  int32_t slot;
  if (!free_handles_.empty()) {
    slot = free_handles_.back();
    free_handles_.pop_back();
  } else {
    slot = static_cast<int32_t>(handles_.size());
    handles_.emplace_back();
    handles_.back().gen = 0;
  }
  Handle& h = handles_[slot];
  h.gen += 1;
  if (h.gen == 0) h.gen = 1;
  h.tip = tip;
  h.live = true;
  *out = (static_cast<uint64_t>(h.gen) << 32) | static_cast<uint32_t>(slot);
  return TKV_OK;
}

int Tree::resolve(tkv_seq s, int32_t* tip) const {
  const uint32_t slot = static_cast<uint32_t>(s & 0xffffffffu);
  const uint32_t gen = static_cast<uint32_t>(s >> 32);
  if (s == 0 || slot >= handles_.size()) return TKV_E_BADSEQ;
  const Handle& h = handles_[slot];
  if (!h.live || h.gen != gen) return TKV_E_BADSEQ;
  *tip = h.tip;
  return TKV_OK;
}

int Tree::seq_new(tkv_seq* out) {
  if (!out) return TKV_E_INVAL;
  try {
    make_room(handles_, 1);
    make_room(nodes_, 1);
    const int32_t n = new_node();
    nodes_[n].refs = 1;
    nodes_[n].nhandles = 1;
    new_handle(n, out);
  } catch (const std::bad_alloc&) {
    return TKV_E_NOMEM;
  }
  ++epoch_;
  ++shape_epoch_;
  return TKV_OK;
}

int Tree::fork(tkv_seq parent, int32_t n, tkv_seq* out) {
  if (n < 1 || !out) return TKV_E_INVAL;
  int32_t tip;
  if (int rc = resolve(parent, &tip)) return rc;
  try {
    // Make room first so that nothing below can fail half-way.
    const size_t need = n > (int32_t)free_handles_.size() ? n - free_handles_.size() : 0;
    make_room(handles_, need);
  } catch (const std::bad_alloc&) {
    return TKV_E_NOMEM;
  }
  Node& t = nodes_[tip];
  t.frozen = true;  // the shared tail is never written again
  t.refs += n;
  t.nhandles += n;
  for (int32_t i = 0; i < n; ++i) new_handle(tip, &out[i]);
  ++epoch_;
  ++shape_epoch_;
  return TKV_OK;
}

int Tree::release(tkv_seq s) {
  int32_t tip;
  if (int rc = resolve(s, &tip)) return rc;
  const uint32_t slot = static_cast<uint32_t>(s & 0xffffffffu);
  Handle& h = handles_[slot];
  h.live = false;
  h.tip = -1;
  free_handles_.push_back(static_cast<int32_t>(slot));
  int32_t id = tip;
  nodes_[id].nhandles -= 1;
  nodes_[id].refs -= 1;
  while (id >= 0 && nodes_[id].refs == 0) {
    const int32_t p = nodes_[id].parent;
    free_node(id);
    if (p >= 0) nodes_[p].refs -= 1;
    id = p;
  }
  ++epoch_;
  ++shape_epoch_;
  return TKV_OK;
}

int Tree::truncate(tkv_seq s, int64_t new_len) {
  int32_t tip;
  if (int rc = resolve(s, &tip)) return rc;
  Node& t = nodes_[tip];
  const int64_t len = t.base + t.ntok;
  if (new_len < 0 || new_len > len) return TKV_E_RANGE;
  if (new_len == len) return TKV_OK;
  // Only tokens in the handle's own, never-forked tip node may go.
  if (t.frozen || new_len < t.base) return TKV_E_SHARED;
  const int64_t keep_tok = new_len - t.base;
  const size_t keep_blk = static_cast<size_t>((keep_tok + 15) / 16);
  for (size_t i = keep_blk; i < t.blocks.size(); ++i) {
    pool_.give(t.blocks[i]);
    block_owner_[t.blocks[i]] = -1;
    ++counters.blocks_freed;
  }
  t.blocks.resize(keep_blk);
  t.ntok = keep_tok;
  ++epoch_;
  ++shape_epoch_;
  return TKV_OK;
}

int Tree::append_need(tkv_seq s, int32_t ntok, int64_t* blocks) const {
  if (ntok < 1 || !blocks) return TKV_E_INVAL;
  int32_t tip;
  if (int rc = resolve(s, &tip)) return rc;
  const Node& t = nodes_[tip];
  const int32_t room = t.frozen ? 0 : (t.blocks.empty() ? 0 : 16 - t.tail_valid());
  *blocks = (std::max<int64_t>(0, (int64_t)ntok - room) + 15) / 16;
  return TKV_OK;
}

int Tree::append(tkv_seq s, int32_t ntok, Placement* pl) {
  if (ntok < 1 || !pl) return TKV_E_INVAL;
  int32_t tip;
  if (int rc = resolve(s, &tip)) return rc;
  const bool need_node = nodes_[tip].frozen;
  const int32_t room = need_node ? 0 : (nodes_[tip].blocks.empty() ? 0 : 16 - nodes_[tip].tail_valid());
  const int64_t rest = std::max<int64_t>(0, (int64_t)ntok - room);
  const int64_t need = (rest + 15) / 16;
  if (need > pool_.num_free()) return TKV_E_NOMEM;
  try {
    pl->blocks.clear();
    pl->blocks.reserve(need + 1);
    make_room(nodes_, 1);
    make_room(nodes_[tip].blocks, static_cast<size_t>(need));
  } catch (const std::bad_alloc&) {
    return TKV_E_NOMEM;
  }
  int32_t id = tip;
  last_made_node_ = false;
  if (need_node) {
    const int32_t c = new_node();
    Node& p = nodes_[tip];
    Node& n = nodes_[c];
    n.parent = tip;
    n.depth = p.depth + 1;
    n.base = p.base + p.ntok;
    n.refs = 1;
    n.nhandles = 1;
    // the handle moves from p to its new child: p gains a child, loses a handle
    p.nhandles -= 1;
    const uint32_t slot = static_cast<uint32_t>(s & 0xffffffffu);
    handles_[slot].tip = c;
    id = c;
    last_made_node_ = true;
    try {
      n.blocks.reserve(need);
    } catch (const std::bad_alloc&) {
      // cannot happen in practice; undo the node to keep the strong guarantee
      p.nhandles += 1;
      handles_[slot].tip = tip;
      free_node(c);
      return TKV_E_NOMEM;
    }
  }
  Node& n = nodes_[id];
  pl->first_slot = room > 0 ? n.tail_valid() : 0;
  if (room > 0) pl->blocks.push_back(n.blocks.back());
  for (int64_t i = 0; i < need; ++i) {
    const int32_t b = pool_.take();
    block_owner_[b] = id;
    n.blocks.push_back(b);
    pl->blocks.push_back(b);
    ++counters.blocks_taken;
  }
  n.ntok += ntok;
  ++epoch_;
  if (need_node || need > 0) ++shape_epoch_;
  return TKV_OK;
}

void Tree::undo_append(tkv_seq s, int32_t ntok, const Placement& pl, bool made_node) {
  int32_t tip;
  if (resolve(s, &tip)) return;
  Node& n = nodes_[tip];
  const size_t fresh = pl.blocks.size() - (pl.first_slot > 0 ? 1 : 0);
  for (size_t i = 0; i < fresh; ++i) {
    const int32_t b = n.blocks.back();
    n.blocks.pop_back();
    pool_.give(b);
    block_owner_[b] = -1;
    --counters.blocks_taken;
  }
  n.ntok -= ntok;
  if (made_node) {
    const int32_t p = n.parent;
    const uint32_t slot = static_cast<uint32_t>(s & 0xffffffffu);
    handles_[slot].tip = p;
    nodes_[p].nhandles += 1;
    n.reset();
    free_nodes_.push_back(tip);
    --counters.nodes_created;
  }
  ++epoch_;
  ++shape_epoch_;
}

int Tree::seq_len(tkv_seq s, int64_t* len) const {
  if (!len) return TKV_E_INVAL;
  int32_t tip;
  if (int rc = resolve(s, &tip)) return rc;
  *len = nodes_[tip].base + nodes_[tip].ntok;
  return TKV_OK;
}

int Tree::own_last_token(tkv_seq s, int32_t* block, int32_t* slot) const {
  if (!block || !slot) return TKV_E_INVAL;
  int32_t id;
  if (int rc = resolve(s, &id)) return rc;
  const Node& t = nodes_[id];
  if (t.ntok == 0 || t.frozen) return t.base + t.ntok == 0 ? TKV_E_EMPTY : TKV_E_SHARED;
  *block = t.blocks.back();
  *slot = t.tail_valid() - 1;
  return TKV_OK;
}

int Tree::block_table(tkv_seq s, int32_t* ids, int32_t* valid, int32_t cap, int32_t* n) const {
  if (!n) return TKV_E_INVAL;
  int32_t tip;
  if (int rc = resolve(s, &tip)) return rc;
  int64_t total = 0;
  for (int32_t id = tip; id >= 0; id = nodes_[id].parent) total += nodes_[id].blocks.size();
  *n = static_cast<int32_t>(total);
  if (total > cap) return TKV_E_RANGE;
  if (total > 0 && (!ids || !valid)) return TKV_E_INVAL;
  int64_t at = total;
  for (int32_t id = tip; id >= 0; id = nodes_[id].parent) {
    const Node& nd = nodes_[id];
    const int64_t nb = nd.blocks.size();
    at -= nb;
    for (int64_t i = 0; i < nb; ++i) {
      ids[at + i] = nd.blocks[i];
      valid[at + i] = (i == nb - 1) ? nd.tail_valid() : 16;
    }
  }
  return TKV_OK;
}

int Tree::block_refcounts(int32_t* rc) const {
  if (!rc) return TKV_E_INVAL;
  // handles in each node's subtree, accumulated bottom-up by depth
  std::vector<int32_t> order, sub;
  try {
    order.reserve(nodes_.size());
    sub.assign(nodes_.size(), 0);
  } catch (const std::bad_alloc&) {
    return TKV_E_NOMEM;
  }
  for (int32_t i = 0; i < (int32_t)nodes_.size(); ++i)
    if (nodes_[i].live) order.push_back(i);
  std::sort(order.begin(), order.end(),
            [&](int32_t a, int32_t b) { return nodes_[a].depth > nodes_[b].depth; });
  for (int32_t id : order) {
    sub[id] += nodes_[id].nhandles;
    if (nodes_[id].parent >= 0) sub[nodes_[id].parent] += sub[id];
  }
  for (int32_t b = 0; b < pool_.size(); ++b) rc[b] = block_owner_[b] >= 0 ? sub[block_owner_[b]] : 0;
  return TKV_OK;
}

int Tree::block_refcount(int32_t b, int32_t* rc) const {
  if (!rc) return TKV_E_INVAL;
  if (b < 0 || b >= pool_.size()) return TKV_E_RANGE;
  const int32_t owner = block_owner_[b];
  if (owner < 0) {
    *rc = 0;
    return TKV_OK;
  }
  // count live handles whose path passes through the owner
  int32_t count = 0;
  for (const Handle& h : handles_) {
    if (!h.live) continue;
    for (int32_t id = h.tip; id >= 0; id = nodes_[id].parent)
      if (id == owner) {
        ++count;
        break;
      }
  }
  *rc = count;
  return TKV_OK;
}

}  // namespace tkv
