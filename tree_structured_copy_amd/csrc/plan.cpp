#include "plan.h"

#include <algorithm>
#include <cstddef>
#include <cstring>
#include <new>

namespace tkv {

namespace {

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

void Plan::layout() {
  size_t o = 0;
  off_items = o;        o = align256(o + items.size() * sizeof(DevItem));
  off_gq = o;           o = align256(o + gq.size() * sizeof(int32_t));
  off_gqpos = o;        o = align256(o + gqpos.size() * sizeof(int32_t));
  off_blocks = o;       o = align256(o + blocks.size() * sizeof(DevBlock));
  off_parts = o;        o = align256(o + parts.size() * sizeof(DevPart));
  off_merge = o;        o = align256(o + merge.size() * sizeof(DevMerge));
  bytes = o;
}

namespace {

// memcpy of a list that may be empty (an empty vector's data() may be null,
// which memcpy may not be given even for zero bytes)
template <class T, class A>
void put(char* dst, const std::vector<T, A>& v) {
  if (!v.empty()) std::memcpy(dst, v.data(), v.size() * sizeof(T));
}

}  // namespace

void Plan::serialise(void* dst) const {
  char* p = static_cast<char*>(dst);
  put(p + off_items, items);
  put(p + off_gq, gq);
  put(p + off_gqpos, gqpos);
  put(p + off_blocks, blocks);
  put(p + off_parts, parts);
  put(p + off_merge, merge);
}

void Plan::reset() {
  items.clear();
  groups.clear();
  gq.clear();
  gqpos.clear();
  blocks.clear();
  parts.clear();
  merge.clear();
  for (int c = 0; c <= kKernelClasses; ++c) bucket_begin[c] = 0;
  for (int c = 0; c < kKernelClasses; ++c) {
    bucket_max_blocks[c] = 0;
    bucket_blocks[c] = 0;
  }
  nqueries = 0;
  partial_slots = 0;
  any_merge = false;
  causal = false;
  unique_blocks = 0;
  unique_tokens = 0;
  tail_entry.clear();
  tail_node.clear();
  gq_node.clear();
  gq_back.clear();
  open_nodes.clear();
  closed_tokens = 0;
  off_items = off_gq = off_gqpos = off_blocks = off_parts = off_merge = bytes = 0;
}

namespace {

// Clears the tree-node -> local-node map on every way out of build_plan, so
// the scratch map is all -1 again for the next call.
struct LocReset {
  PlanScratch& s;
  ~LocReset() {
    for (int32_t id : s.lnode) s.loc[id] = -1;
    s.lnode.clear();
  }
};

}  // namespace

int build_plan(const Tree& tree, const tkv_seq* seqs, const int32_t* nq, int32_t nseq,
               int32_t q_per_kv, int32_t num_kv_heads, const PlanOptions& opt, Plan* out,
               PlanScratch* scratch) {
  if (!seqs || nseq < 1 || !out || q_per_kv < 1 || q_per_kv > kMaxRows) return TKV_E_INVAL;
  PlanScratch local;
  PlanScratch& S = scratch ? *scratch : local;
  try {
    // 1. handles and queries
    S.tip.resize(nseq);
    S.qn.resize(nseq);
    S.qbase.resize(nseq);
    S.len.resize(nseq);
    int64_t total_q = 0;
    for (int32_t i = 0; i < nseq; ++i) {
      if (int rc = tree.resolve(seqs[i], &S.tip[i])) return rc;
      const Node& t = tree.node(S.tip[i]);
      S.len[i] = t.base + t.ntok;
      S.qn[i] = nq ? nq[i] : 1;
      if (S.len[i] == 0) return TKV_E_EMPTY;
      if (S.qn[i] < 1 || S.qn[i] > S.len[i] || S.len[i] > INT32_MAX) return TKV_E_RANGE;
      S.qbase[i] = static_cast<int32_t>(total_q);
      total_q += S.qn[i];
      if (total_q > INT32_MAX / 4) return TKV_E_RANGE;
    }

    // 2. local tree over the union of the paths: nodes in order of discovery,
    //    their handles and children as index ranges (children by node id)
    if (static_cast<int32_t>(S.loc.size()) < tree.node_capacity()) S.loc.resize(tree.node_capacity(), -1);
    S.lnode.clear();
    S.lparent.clear();
    LocReset reset_loc{S};
    auto& loc = S.loc;
    for (int32_t i = 0; i < nseq; ++i) {
      int32_t prev = -1;
      for (int32_t id = S.tip[i]; id >= 0; id = tree.node(id).parent) {
        if (loc[id] >= 0) {
          if (prev >= 0) S.lparent[prev] = loc[id];
          break;
        }
        loc[id] = static_cast<int32_t>(S.lnode.size());
        S.lnode.push_back(id);
        S.lparent.push_back(-1);
        if (prev >= 0) S.lparent[prev] = loc[id];
        prev = loc[id];
      }
    }
    const int32_t nl = static_cast<int32_t>(S.lnode.size());
    S.hbeg.assign(nl + 1, 0);
    for (int32_t i = 0; i < nseq; ++i) ++S.hbeg[loc[S.tip[i]] + 1];
    for (int32_t k = 0; k < nl; ++k) S.hbeg[k + 1] += S.hbeg[k];
    S.cursor.assign(S.hbeg.begin(), S.hbeg.end() - 1);
    S.hlist.resize(nseq);
    for (int32_t i = 0; i < nseq; ++i) S.hlist[S.cursor[loc[S.tip[i]]]++] = i;
    S.roots.clear();
    S.cbeg.assign(nl + 1, 0);
    for (int32_t k = 0; k < nl; ++k) {
      if (S.lparent[k] >= 0) ++S.cbeg[S.lparent[k] + 1];
      else S.roots.push_back(k);
    }
    for (int32_t k = 0; k < nl; ++k) S.cbeg[k + 1] += S.cbeg[k];
    S.cursor.assign(S.cbeg.begin(), S.cbeg.end() - 1);
    S.child.resize(S.cbeg[nl]);
    for (int32_t k = 0; k < nl; ++k)
      if (S.lparent[k] >= 0) S.child[S.cursor[S.lparent[k]]++] = k;
    auto by_node = [&](int32_t a, int32_t b) { return S.lnode[a] < S.lnode[b]; };
    std::sort(S.roots.begin(), S.roots.end(), by_node);
    for (int32_t k = 0; k < nl; ++k)
      if (S.cbeg[k + 1] - S.cbeg[k] > 1) std::sort(S.child.begin() + S.cbeg[k], S.child.begin() + S.cbeg[k + 1], by_node);

    // DFS preorder (children in node order), then subtree query counts in
    // reverse preorder, where every node comes after its descendants
    S.pre.resize(nl);
    S.by_pre.resize(nl);
    {
      int32_t pre = 0;
      auto& st = S.st;
      st.clear();
      for (int32_t r : S.roots) {
        st.push_back(r);
        while (!st.empty()) {
          const int32_t k = st.back();
          st.pop_back();
          S.pre[k] = pre;
          S.by_pre[pre++] = k;
          for (int32_t c = S.cbeg[k + 1] - 1; c >= S.cbeg[k]; --c) st.push_back(S.child[c]);
        }
      }
    }
    S.qcount.assign(nl, 0);
    for (int32_t p = nl - 1; p >= 0; --p) {
      const int32_t k = S.by_pre[p];
      for (int32_t x = S.hbeg[k]; x < S.hbeg[k + 1]; ++x) S.qcount[k] += S.qn[S.hlist[x]];
      if (S.lparent[k] >= 0) S.qcount[S.lparent[k]] += S.qcount[k];
    }

    // 3. groups: subtrees with <= qg queries become units; units of one tree are
    //    packed in DFS order up to qg queries.  Units are consecutive runs of
    //    one query array, so a group is a run of it too.
    const int32_t rows = std::max(16, std::min<int32_t>(opt.max_rows, kMaxRows));
    const int32_t qg = std::max(1, std::min(kMaxGroupQueries, rows / q_per_kv));
    auto& uq = S.uq;
    uq.clear();
    auto queries_of_handle = [&](int32_t h) {
      for (int32_t k = 0; k < S.qn[h]; ++k)
        uq.push_back({h, S.qbase[h] + k, static_cast<int32_t>(S.len[h] - S.qn[h] + k)});
    };
    S.gbeg.clear();
    S.gsize.clear();
    S.groot.clear();
    {
      auto& st = S.st;
      auto& sub = S.sub;
      auto& ub = S.ub;
      for (size_t r = 0; r < S.roots.size(); ++r) {
        ub.clear();
        st.push_back(S.roots[r]);
        while (!st.empty()) {
          const int32_t k = st.back();
          st.pop_back();
          if (S.qcount[k] <= qg) {
            const size_t u0 = uq.size();
            sub.push_back(k);
            while (!sub.empty()) {
              const int32_t s = sub.back();
              sub.pop_back();
              for (int32_t x = S.hbeg[s]; x < S.hbeg[s + 1]; ++x) queries_of_handle(S.hlist[x]);
              for (int32_t c = S.cbeg[s + 1] - 1; c >= S.cbeg[s]; --c) sub.push_back(S.child[c]);
            }
            if (uq.size() > u0) ub.push_back(static_cast<int32_t>(u0));
          } else {
            const size_t o0 = uq.size();
            for (int32_t x = S.hbeg[k]; x < S.hbeg[k + 1]; ++x) queries_of_handle(S.hlist[x]);
            for (size_t a = o0; a < uq.size(); a += qg) ub.push_back(static_cast<int32_t>(a));
            for (int32_t c = S.cbeg[k + 1] - 1; c >= S.cbeg[k]; --c) st.push_back(S.child[c]);
          }
        }
        // unit u of this tree = uq[ub[u] .. ub[u + 1]), the last one ending at uq.size()
        const size_t g_first = S.gbeg.size();
        int32_t cur_begin = 0, cur_size = 0;
        for (size_t u = 0; u < ub.size(); ++u) {
          const int32_t usz = (u + 1 < ub.size() ? ub[u + 1] : static_cast<int32_t>(uq.size())) - ub[u];
          if (cur_size > 0 && cur_size + usz > qg) {
            S.gbeg.push_back(cur_begin);
            S.gsize.push_back(cur_size);
            S.groot.push_back(static_cast<int32_t>(r));
            cur_size = 0;
          }
          if (cur_size == 0) cur_begin = ub[u];
          cur_size += usz;
        }
        if (cur_size > 0) {
          S.gbeg.push_back(cur_begin);
          S.gsize.push_back(cur_size);
          S.groot.push_back(static_cast<int32_t>(r));
        }
        // The packing leaves the tree's last group with what remains (a
        // 40-way fork: 32 queries, then 8).  The last two groups take the unit
        // boundary that splits their queries most evenly instead (20 and 20):
        // the same row tiles in all, and groups of one size run in one kernel
        // class rather than an 8-tile launch and a 2-tile one.
        const size_t ng = S.gbeg.size();
        if (ng >= g_first + 2) {
          const int32_t a = S.gbeg[ng - 2], end = S.gbeg[ng - 1] + S.gsize[ng - 1];
          int32_t best = S.gbeg[ng - 1];
          for (size_t u = 0; u < ub.size(); ++u) {
            const int32_t cut = ub[u];
            if (cut <= a || cut >= end || cut - a > qg || end - cut > qg) continue;
            if (std::max(cut - a, end - cut) < std::max(best - a, end - best)) best = cut;
          }
          S.gsize[ng - 2] = best - a;
          S.gbeg[ng - 1] = best;
          S.gsize[ng - 1] = end - best;
        }
      }
    }

    // 4. per-group block lists.  A large group (8+ row tiles) whose blocks are
    //    partly narrow -- seen only by queries that one row tile holds, as the
    //    deep, private nodes of a search tree are -- keeps its widely shared
    //    blocks and hands each narrow node to a one-tile subgroup of its
    //    queries: a large group costs row-tile work on every block it reads,
    //    a one-tile group about its memory time.  A query then has partial
    //    records in both groups, merged afterwards.
    // The LDS-staged kernels spend, on a block, its memory time plus the math
    // of every row tile with a query that sees it (a wave skips a block none
    // of its rows sees).  Their groups are chunked by cost,
    // kBlockCost + (row tiles that see the block - 1) per block, so that a
    // chunk of a widely shared root is shorter than one of private leaves,
    // and a group's share of its class's items follows its cost.
    constexpr int64_t kBlockCost = kPlanBlockCost;
    // tile bits of the queries of one byte of a visibility mask, by byte
    // position (made once per query heads per KV head: the scratch keeps it)
    auto& tile_of_byte = S.tile_of_byte;
    if (S.tile_of_byte_qpk != q_per_kv) {
      tile_of_byte.assign(8 * 256, 0);
      for (int32_t pb = 0; pb < 8; ++pb)
        for (int32_t v = 1; v < 256; ++v) {
          uint32_t t = 0;
          for (int32_t bit = 0; bit < 8; ++bit)
            if ((v >> bit) & 1) {
              const int32_t j = 8 * pb + bit;
              if (j * q_per_kv >= kMaxRows) break;  // no group holds query j
              for (int32_t tl = (j * q_per_kv) >> 4; tl <= (j * q_per_kv + q_per_kv - 1) >> 4; ++tl)
                t |= 1u << tl;
            }
          tile_of_byte[pb * 256 + v] = t;
        }
      S.tile_of_byte_qpk = q_per_kv;
    }
    auto tiles_seeing = [&](uint64_t m) {
      uint32_t t = 0;
      for (int32_t pb = 0; m; ++pb, m >>= 8) t |= tile_of_byte[pb * 256 + static_cast<int32_t>(m & 0xff)];
      return __builtin_popcount(t);
    };
    auto block_cost = [&](const DevBlock& b) -> int64_t { return kBlockCost + tiles_seeing(b.mask) - 1; };
    Plan& P = *out;
    P.reset();
    P.nqueries = static_cast<int32_t>(total_q);
    P.causal = nq != nullptr;
    // groups made, in order: block range, tree, whether its queries have records elsewhere too
    S.go_begin.clear();
    S.go_count.clear();
    S.go_root.clear();
    S.go_partials.clear();
    S.go_cost.clear();
    S.go_mask.clear();
    // the (group, index in group) of each query's at most two groups: its own
    // and possibly one cascade subgroup of it
    S.qm_n.assign(total_q, 0);
    S.qm_g.resize(2 * total_q);
    S.qm_j.resize(2 * total_q);
    S.mask.assign(nl, 0);
    S.emitted.assign(nl, 0);
    auto& mask = S.mask;
    auto& touched = S.touched;
    const int32_t sub = std::max(1, 16 / q_per_kv);  // queries of a one-tile subgroup
    auto emit_group = [&](const PlanQuery* qs, int32_t n, int32_t root, bool partials) {
      const int32_t gi = static_cast<int32_t>(P.groups.size());
      DevGroup g;
      g.q_begin = static_cast<int32_t>(P.gq.size());
      g.nq = n;
      g.min_pos = INT32_MAX;
      g.pad1 = 0;
      // sized once, then written: element-wise push_back costs several times more
      const size_t at0 = P.gq.size();
      P.gq.resize(at0 + n);
      P.gqpos.resize(at0 + n);
      P.gq_node.resize(at0 + n);
      P.gq_back.resize(at0 + n);
      for (int32_t j = 0; j < n; ++j) {
        const int32_t q = qs[j].global;
        P.gq[at0 + j] = q;
        P.gqpos[at0 + j] = qs[j].pos;
        P.gq_node[at0 + j] = S.tip[qs[j].handle];
        P.gq_back[at0 + j] = static_cast<int32_t>(S.len[qs[j].handle] - qs[j].pos);
        g.min_pos = std::min(g.min_pos, qs[j].pos);
        const int32_t at = 2 * q + S.qm_n[q]++;
        S.qm_g[at] = gi;
        S.qm_j[at] = j;
      }
      P.groups.push_back(g);
      S.go_begin.push_back(static_cast<int32_t>(P.blocks.size()));
      S.go_count.push_back(0);
      S.go_root.push_back(root);
      S.go_partials.push_back(partials ? 1 : 0);
      S.go_cost.push_back(0);
      S.go_mask.push_back(0);
    };
    // a node's blocks, once per group that reads it; the statistics count each node once
    auto emit_node = [&](int32_t k, uint64_t m) {
      const Node& nd = tree.node(S.lnode[k]);
      const int32_t nb = static_cast<int32_t>(nd.blocks.size());
      const size_t at = P.blocks.size();
      P.blocks.resize(at + nb);
      DevBlock* out = P.blocks.data() + at;
      const int32_t* ids = nd.blocks.data();
      const int32_t pos0 = static_cast<int32_t>(nd.base);
      for (int32_t b = 0; b < nb; ++b) {
        out[b].id = ids[b];
        out[b].pos = pos0 + 16 * b;
        out[b].valid = 16;
        out[b].pad = 0;
        out[b].mask = m;
      }
      if (nb > 0) {
        out[nb - 1].valid = nd.tail_valid();
        // the group's cost and query mask, one lookup per node (its blocks share the mask)
        S.go_cost.back() += static_cast<int64_t>(nb) * (kBlockCost + tiles_seeing(m) - 1);
        S.go_mask.back() |= m;
      }
      if (!nd.frozen && nb > 0) {
        P.tail_entry.push_back(static_cast<int32_t>(P.blocks.size()) - 1);
        P.tail_node.push_back(S.lnode[k]);
      }
      if (!S.emitted[k]) {
        S.emitted[k] = 1;
        P.unique_blocks += nb;
        P.unique_tokens += nd.ntok;
        if (nd.frozen) P.closed_tokens += nd.ntok;
        else P.open_nodes.push_back(S.lnode[k]);
      }
    };
    auto close_group = [&]() { S.go_count.back() = static_cast<int32_t>(P.blocks.size()) - S.go_begin.back(); };
    // the subgroup a node's queries fit in, or -1
    auto narrow = [&](uint64_t m) {
      const int32_t lo = __builtin_ctzll(m), hi = 63 - __builtin_clzll(m);
      return lo / sub == hi / sub ? lo / sub : -1;
    };
    for (size_t g0 = 0; g0 < S.gbeg.size(); ++g0) {
      const PlanQuery* qs = uq.data() + S.gbeg[g0];
      const int32_t n = S.gsize[g0];
      touched.clear();
      for (int32_t j = 0; j < n;) {
        // a handle's queries are consecutive and see the same nodes: one walk
        // up its path per handle, with all their bits
        const int32_t h = qs[j].handle;
        uint64_t bits = 0;
        int32_t j1 = j;
        for (; j1 < n && qs[j1].handle == h; ++j1) bits |= 1ull << j1;
        for (int32_t k = loc[S.tip[h]]; k >= 0; k = S.lparent[k]) {
          if (!mask[k]) touched.push_back(k);
          mask[k] |= bits;
        }
        j = j1;
      }
      std::sort(touched.begin(), touched.end(), [&](int32_t a, int32_t b) { return S.pre[a] < S.pre[b]; });
      bool cascade = false;
      const int32_t ntouch = static_cast<int32_t>(touched.size());
      if (opt.cascade && (n * q_per_kv + 15) / 16 >= 8 && n > sub) {
        // each node's subgroup (or -1) once, and the narrow nodes bucketed by
        // subgroup in touched order
        const int32_t nsub = (n + sub - 1) / sub;
        S.nar.resize(ntouch);
        S.sbeg.assign(nsub + 1, 0);
        int64_t all = 0, thin = 0;
        for (int32_t i = 0; i < ntouch; ++i) {
          const int32_t k = touched[i];
          const int64_t nb = static_cast<int64_t>(tree.node(S.lnode[k]).blocks.size());
          S.nar[i] = narrow(mask[k]);
          all += nb;
          if (S.nar[i] >= 0) {
            thin += nb;
            ++S.sbeg[S.nar[i] + 1];
          }
        }
        cascade = thin * 8 >= all && thin > 0;
        if (cascade) {
          for (int32_t t = 0; t < nsub; ++t) S.sbeg[t + 1] += S.sbeg[t];
          S.cursor.assign(S.sbeg.begin(), S.sbeg.end() - 1);
          S.sorder.resize(S.sbeg[nsub]);
          for (int32_t i = 0; i < ntouch; ++i)
            if (S.nar[i] >= 0) S.sorder[S.cursor[S.nar[i]]++] = i;
        }
      }
      emit_group(qs, n, S.groot[g0], cascade);
      for (int32_t i = 0; i < ntouch; ++i)
        if (!cascade || S.nar[i] < 0) emit_node(touched[i], mask[touched[i]]);
      close_group();
      if (cascade) {
        for (int32_t t = 0; t * sub < n; ++t) {
          if (S.sbeg[t + 1] == S.sbeg[t]) continue;
          emit_group(qs + t * sub, std::min(sub, n - t * sub), S.groot[g0], true);
          for (int32_t x = S.sbeg[t]; x < S.sbeg[t + 1]; ++x) {
            const int32_t k = touched[S.sorder[x]];
            emit_node(k, mask[k] >> (t * sub));
          }
          close_group();
        }
      }
      for (int32_t k : touched) mask[k] = 0;
    }
    const int32_t ngroups = static_cast<int32_t>(P.groups.size());

    // 5. split-K chunking and items.  The kernel classes of a call do not
    //    share the GPU well (a class's workgroups take whole CUs' registers or
    //    LDS, and side-stream joins cost more than the overlap gains), so each
    //    class is cut to fill the GPU on its own: about target_wgs / Hkv items
    //    (one round of workgroups), shared among its groups in proportion to
    //    their cost (below).  A chunk stays long
    //    next to its partial record: at least min_chunk blocks for the
    //    register-tile classes, whose time is their memory time, and a quarter
    //    of that for the LDS-staged classes (3+ row tiles), whose time per
    //    block is several times longer; and at most kRowsMaxItemBlocks.
    //    With groups of at most 8 row tiles, every LDS-staged class below the
    //    largest one present runs in that class's kernel (its extra waves
    //    idle): one launch, one ramp and one tail instead of several, each
    //    class filling the GPU alone (a search tree whose groups came out of
    //    6 and 8 tiles: 60 -> 37 us).  Below a 16-tile class (groups of up to
    //    256 rows) only a class with less work (blocks x row tiles) than that
    //    class joins it: a 16-tile workgroup holds a CU alone.
    auto& gclass = S.gclass;
    gclass.resize(ngroups);
    int64_t class_work[kKernelClasses] = {0, 0, 0, 0, 0, 0};
    for (int32_t gi = 0; gi < ngroups; ++gi) {
      const int32_t tiles = (P.groups[gi].nq * q_per_kv + 15) / 16;
      gclass[gi] = static_cast<int8_t>(kernel_class(tiles));
      class_work[gclass[gi]] += static_cast<int64_t>(S.go_count[gi]) * tiles;
    }
    int top = -1;
    for (int c = 2; c < kKernelClasses; ++c)
      if (class_work[c] > 0) top = c;
    if (top > 2)
      for (int32_t gi = 0; gi < ngroups; ++gi)
        if (gclass[gi] >= 2 && gclass[gi] < top && (top <= 4 || class_work[gclass[gi]] < class_work[top]))
          gclass[gi] = top;
    auto class_of = [&](int32_t gi) { return static_cast<int>(gclass[gi]); };
    auto& gcost = S.gcost;
    gcost.assign(ngroups, 0);
    int64_t class_cost[kKernelClasses] = {0, 0, 0, 0, 0, 0};
    int64_t class_blocks[kKernelClasses] = {0, 0, 0, 0, 0, 0};
    for (int32_t gi = 0; gi < ngroups; ++gi) {
      const int cls = class_of(gi);
      const int32_t nb = S.go_count[gi];
      gcost[gi] = cls >= 2 ? S.go_cost[gi] : nb;
      class_cost[cls] += gcost[gi];
      class_blocks[cls] += nb;
    }
    const int64_t class_items = std::max<int64_t>(1, std::max<int32_t>(1, opt.target_wgs) / num_kv_heads);
    auto want_of = [&](int cls) -> int64_t {
      // the 4- and 8-tile LDS-staged shapes fit two workgroups per CU, and
      // two per CU stream faster than one with a deeper ring; the 6-tile
      // shape's workgroups pair two KV heads: twice the items either way
      // (a 24-branch fork's 6-tile groups: 122 -> 83 us)
      return (opt.two_per_cu && cls >= 2 && cls <= 4) ? 2 * class_items : class_items;
    };
    auto most_of = [&](int32_t gi) -> int64_t {
      const int cls = class_of(gi);
      // a class too small to give every item its floor of blocks (a few
      // queries over a few thousand tokens) is latency-bound, not
      // bandwidth-bound: its floor drops to what fills the GPU, at least 4
      const int64_t base = std::max<int32_t>(1, cls < 2 ? opt.min_chunk : opt.min_chunk / 4);
      const int64_t floor =
          std::max<int64_t>(1, std::min(base, std::max<int64_t>(4, class_blocks[cls] / want_of(cls))));
      return std::max<int64_t>(1, S.go_count[gi] / floor);
    };
    // Chunks per group: the group's share of its class's items by cost,
    // rounded down; the items that leaves go one each to the groups with the
    // largest remainders, so that a class fills one round of workgroups.  A
    // chunk stays at least the floor above and at most kRowsMaxItemBlocks.
    auto& gchunks = S.gchunks;
    auto& gfrac = S.gfrac;
    gchunks.assign(ngroups, 1);
    gfrac.assign(ngroups, -1.0);
    int64_t class_chunks[kKernelClasses] = {0, 0, 0, 0, 0, 0};
    for (int32_t gi = 0; gi < ngroups; ++gi) {
      const int cls = class_of(gi);
      const int64_t nb = S.go_count[gi];
      if (nb == 0) continue;
      const double ideal = static_cast<double>(gcost[gi]) * static_cast<double>(want_of(cls)) /
                           static_cast<double>(std::max<int64_t>(1, class_cost[cls]));
      const int64_t most = most_of(gi);
      const int64_t least = (nb + kRowsMaxItemBlocks - 1) / kRowsMaxItemBlocks;
      int64_t nc = std::min(static_cast<int64_t>(ideal), most);
      nc = std::max<int64_t>(std::max<int64_t>(nc, least), 1);
      gchunks[gi] = static_cast<int32_t>(nc);
      if (nc < most && static_cast<double>(nc) < ideal) gfrac[gi] = ideal - static_cast<double>(nc);
      class_chunks[cls] += nc;
    }
    for (int cls = 0; cls < kKernelClasses; ++cls) {
      for (int64_t left = want_of(cls) - class_chunks[cls]; left > 0; --left) {
        int32_t best = -1;
        for (int32_t gi = 0; gi < ngroups; ++gi)
          if (class_of(gi) == cls && gfrac[gi] > 0.0 && (best < 0 || gfrac[gi] > gfrac[best])) best = gi;
        if (best < 0) break;
        ++gchunks[best];
        gfrac[best] = -1.0;  // one extra chunk per group
      }
    }
    auto& cut = S.cut;
    auto& tmp = S.tmp;
    tmp.clear();
    int64_t slots = 0;
    for (int32_t gi = 0; gi < ngroups; ++gi) {
      const int32_t nb = S.go_count[gi];
      if (nb == 0) continue;
      const int32_t nc = gchunks[gi];
      const int32_t tiles = class_of(gi);
      // chunk c is blocks [cut[c], cut[c + 1]) of the group's list
      cut.assign(nc + 1, nb);
      cut[0] = 0;
      bool weighted = false;
      if (tiles >= 2 && nc > 1) {
        const DevBlock* gb = P.blocks.data() + S.go_begin[gi];
        const uint64_t full = P.groups[gi].nq >= 64 ? ~0ull : ((1ull << P.groups[gi].nq) - 1);
        for (int32_t b = 0; b < nb && !weighted; ++b) weighted = gb[b].mask != full;
        if (weighted) {
          const int64_t total = gcost[gi];
          int64_t acc = 0;
          int32_t c = 1;
          uint64_t run_mask = gb[0].mask;
          int64_t run_cost = block_cost(gb[0]);
          for (int32_t b = 0; b < nb && c < nc; ++b) {
            if (gb[b].mask != run_mask) {
              run_mask = gb[b].mask;
              run_cost = block_cost(gb[b]);
            }
            acc += run_cost;
            // close chunk c - 1 after block b once it holds its share of the
            // cost, leaving at least one block for each chunk still to come
            if (acc * nc >= total * c && nb - (b + 1) >= nc - c) cut[c++] = b + 1;
          }
          for (; c < nc; ++c) cut[c] = nb - (nc - c);
          // no chunk longer than a staged block list
          for (int32_t k = 0; k < nc && weighted; ++k)
            if (cut[k + 1] - cut[k] > kRowsMaxItemBlocks) weighted = false;
        }
      }
      if (!weighted)
        for (int32_t c = 0; c < nc; ++c) cut[c + 1] = cut[c] + nb / nc + (c < nb % nc ? 1 : 0);
      int32_t at = 0;
      for (int32_t c = 0; c < nc; ++c) {
        const int32_t cnt = cut[c + 1] - cut[c];
        PlanItemTmp t;
        t.it.group = gi;
        t.it.blk_begin = S.go_begin[gi] + at;
        t.it.blk_count = cnt;
        t.it.q_begin = P.groups[gi].q_begin;
        t.it.nq = P.groups[gi].nq;
        t.it.min_pos = P.groups[gi].min_pos;
        t.it.tails = 0;
        t.it.qmask = 0;
        t.it.pad0 = t.it.pad1 = 0;
        if (nc == 1) {
          t.it.qmask = S.go_mask[gi];
        } else {
          for (int32_t b = 0; b < cnt; ++b) t.it.qmask |= P.blocks[S.go_begin[gi] + at + b].mask;
        }
        if (nc == 1 && !S.go_partials[gi]) {
          t.it.part_base = -1;
        } else {
          t.it.part_base = static_cast<int32_t>(slots);
          slots += static_cast<int64_t>(P.groups[gi].nq) * q_per_kv * num_kv_heads;
          if (slots > INT32_MAX) return TKV_E_RANGE;
        }
        t.tiles = tiles;
        t.root = S.go_root[gi];
        t.chunk = c;
        tmp.push_back(t);
        at += cnt;
      }
    }
    P.partial_slots = slots;
    // order: by kernel class; longest items first, so that when a class has
    // more workgroups than the GPU holds at once the ones that start late are
    // short; then items that read the same blocks next to each other (same
    // tree, same chunk index), so the KV heads' workgroups of neighbouring
    // items share L2.  (group, chunk) is unique, so the order is total.
    std::sort(tmp.begin(), tmp.end(), [](const PlanItemTmp& a, const PlanItemTmp& b) {
      if (a.tiles != b.tiles) return a.tiles < b.tiles;
      if (a.it.blk_count != b.it.blk_count) return a.it.blk_count > b.it.blk_count;
      if (a.root != b.root) return a.root < b.root;
      if (a.chunk != b.chunk) return a.chunk < b.chunk;
      return a.it.group < b.it.group;
    });
    const int32_t nitems = static_cast<int32_t>(tmp.size());
    P.items.resize(nitems);
    // the items of each group, in item order
    S.ibeg.assign(ngroups + 1, 0);
    for (int32_t k = 0; k < nitems; ++k) {
      P.items[k] = tmp[k].it;
      ++S.ibeg[tmp[k].it.group + 1];
    }
    for (int32_t g = 0; g < ngroups; ++g) S.ibeg[g + 1] += S.ibeg[g];
    S.cursor.assign(S.ibeg.begin(), S.ibeg.end() - 1);
    S.ilist.resize(nitems);
    for (int32_t k = 0; k < nitems; ++k) S.ilist[S.cursor[tmp[k].it.group]++] = k;
    for (int c = 0; c < kKernelClasses; ++c) {
      int32_t cnt = 0;
      for (const auto& x : tmp) cnt += (x.tiles <= c);
      P.bucket_begin[c + 1] = cnt;
    }
    for (const auto& x : tmp) {
      P.bucket_max_blocks[x.tiles] = std::max(P.bucket_max_blocks[x.tiles], x.it.blk_count);
      P.bucket_blocks[x.tiles] += x.it.blk_count;
    }
    // each item's range of tail blocks (tail_entry is in block-list order)
    for (int32_t k = 0; k < nitems; ++k) {
      DevItem& it = P.items[k];
      const auto b = std::lower_bound(P.tail_entry.begin(), P.tail_entry.end(), it.blk_begin);
      const auto e = std::lower_bound(b, P.tail_entry.end(), it.blk_begin + it.blk_count);
      const int64_t lo = b - P.tail_entry.begin(), cnt = e - b;
      it.tails = (cnt > 0 && lo < 0x10000 && cnt < 0x8000) ? static_cast<int32_t>(lo | (cnt << 16)) : 0;
    }
    // merge records: every partial of a query, in the order its groups were
    // made.  With no partial records at all, every group is one item writing
    // its queries' outputs itself (a cascade subgroup always writes partials),
    // so each query has one direct item and an empty record.
    P.merge.resize(total_q);
    if (slots == 0) {
      std::fill(P.merge.begin(), P.merge.end(), DevMerge{0, 0});
    } else {
      for (int64_t q = 0; q < total_q; ++q) {
        DevMerge m;
        m.p_begin = static_cast<int32_t>(P.parts.size());
        int32_t direct = 0;
        for (int32_t x = 0; x < S.qm_n[q]; ++x) {
          const int32_t g = S.qm_g[2 * q + x], j = S.qm_j[2 * q + x];
          for (int32_t y = S.ibeg[g]; y < S.ibeg[g + 1]; ++y) {
            const int32_t item = S.ilist[y];
            if (P.items[item].part_base < 0) {
              ++direct;
              continue;
            }
            if (!((P.items[item].qmask >> j) & 1ull)) continue;  // sees none of the item's blocks
            P.parts.push_back({P.items[item].part_base + j * q_per_kv * num_kv_heads, item});
          }
        }
        m.p_count = static_cast<int32_t>(P.parts.size()) - m.p_begin;
        if (direct + m.p_count == 0 || (direct > 0 && (direct > 1 || m.p_count > 0))) return TKV_E_INVAL;
        P.merge[q] = m;
        if (m.p_count) P.any_merge = true;
      }
    }
    P.layout();
  } catch (const std::bad_alloc&) {
    return TKV_E_NOMEM;
  }
  return TKV_OK;
}

void patch_plan(const Tree& tree, Plan* plan, std::vector<PlanWord>* changed) {
  Plan& P = *plan;
  auto put = [&](size_t byte_offset, int32_t value) {
    if (changed) changed->push_back({static_cast<uint32_t>(byte_offset / 4), value});
  };
  for (size_t t = 0; t < P.tail_entry.size(); ++t) {
    const int32_t e = P.tail_entry[t];
    const int32_t v = tree.node(P.tail_node[t]).tail_valid();
    if (P.blocks[e].valid != v) {
      P.blocks[e].valid = v;
      put(P.off_blocks + e * sizeof(DevBlock) + offsetof(DevBlock, valid), v);
    }
  }
  for (size_t j = 0; j < P.gq.size(); ++j) {
    const Node& nd = tree.node(P.gq_node[j]);
    const int32_t pos = static_cast<int32_t>(nd.base + nd.ntok - P.gq_back[j]);
    if (P.gqpos[j] != pos) {
      P.gqpos[j] = pos;
      put(P.off_gqpos + j * sizeof(int32_t), pos);
    }
  }
  for (auto& g : P.groups) {
    g.min_pos = INT32_MAX;
    for (int32_t j = g.q_begin; j < g.q_begin + g.nq; ++j) g.min_pos = std::min(g.min_pos, P.gqpos[j]);
  }
  for (size_t i = 0; i < P.items.size(); ++i) {
    DevItem& it = P.items[i];
    const int32_t m = P.groups[it.group].min_pos;
    if (it.min_pos != m) {
      it.min_pos = m;
      put(P.off_items + i * sizeof(DevItem) + offsetof(DevItem, min_pos), m);
    }
  }
  P.unique_tokens = P.closed_tokens;
  for (int32_t id : P.open_nodes) P.unique_tokens += tree.node(id).ntok;
}

}  // namespace tkv
