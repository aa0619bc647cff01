#include "plan.h"

#include <algorithm>
#include <cstring>
#include <new>

namespace tkv {

namespace {

struct LNode {
  int32_t node = -1;    // tree node id
  int32_t parent = -1;  // local index
  int32_t pre = 0;      // DFS preorder index
  int32_t root = 0;     // index of its tree's root in the root list
  int64_t qcount = 0;   // queries in the subtree
  std::vector<int32_t> children;
  std::vector<int32_t> handles;  // batch indices whose tip is this node
};

struct Query {
  int32_t handle;  // batch index
  int32_t global;  // global query index (row of q / out)
  int32_t pos;     // absolute position
};

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

void Plan::serialise(void* dst) const {
  char* p = static_cast<char*>(dst);
  std::memcpy(p + off_items, items.data(), items.size() * sizeof(DevItem));
  std::memcpy(p + off_gq, gq.data(), gq.size() * sizeof(int32_t));
  std::memcpy(p + off_gqpos, gqpos.data(), gqpos.size() * sizeof(int32_t));
  std::memcpy(p + off_blocks, blocks.data(), blocks.size() * sizeof(DevBlock));
  std::memcpy(p + off_parts, parts.data(), parts.size() * sizeof(DevPart));
  std::memcpy(p + off_merge, merge.data(), merge.size() * sizeof(DevMerge));
}

int build_plan(const Tree& tree, const tkv_seq* seqs, const int32_t* nq, int32_t nseq,
               int32_t q_per_kv, int32_t num_kv_heads, const PlanOptions& opt, Plan* out) {
  if (!seqs || nseq < 1 || !out || q_per_kv < 1 || q_per_kv > kMaxRows) return TKV_E_INVAL;
  try {
    // 1. handles and queries
    std::vector<int32_t> tip(nseq), qn(nseq), qbase(nseq);
    std::vector<int64_t> len(nseq);
    int64_t total_q = 0;
    for (int32_t i = 0; i < nseq; ++i) {
      if (int rc = tree.resolve(seqs[i], &tip[i])) return rc;
      const Node& t = tree.node(tip[i]);
      len[i] = t.base + t.ntok;
      qn[i] = nq ? nq[i] : 1;
      if (len[i] == 0) return TKV_E_EMPTY;
      if (qn[i] < 1 || qn[i] > len[i] || len[i] > INT32_MAX) return TKV_E_RANGE;
      qbase[i] = static_cast<int32_t>(total_q);
      total_q += qn[i];
      if (total_q > INT32_MAX / 4) return TKV_E_RANGE;
    }

    // 2. local tree over the union of the paths
    std::vector<int32_t> loc(tree.node_capacity(), -1);
    std::vector<LNode> ln;
    for (int32_t i = 0; i < nseq; ++i) {
      int32_t prev = -1;
      for (int32_t id = tip[i]; id >= 0; id = tree.node(id).parent) {
        if (loc[id] >= 0) {
          if (prev >= 0) ln[prev].parent = loc[id];
          break;
        }
        loc[id] = static_cast<int32_t>(ln.size());
        ln.emplace_back();
        ln.back().node = id;
        if (prev >= 0) ln[prev].parent = loc[id];
        prev = loc[id];
      }
      ln[loc[tip[i]]].handles.push_back(i);
    }
    const int32_t nl = static_cast<int32_t>(ln.size());
    std::vector<int32_t> roots;
    for (int32_t k = 0; k < nl; ++k) {
      if (ln[k].parent >= 0) ln[ln[k].parent].children.push_back(k);
      else roots.push_back(k);
    }
    auto by_node = [&](int32_t a, int32_t b) { return ln[a].node < ln[b].node; };
    std::sort(roots.begin(), roots.end(), by_node);
    for (auto& n : ln) std::sort(n.children.begin(), n.children.end(), by_node);

    // subtree query counts, bottom-up by depth
    {
      std::vector<int32_t> order(nl);
      for (int32_t k = 0; k < nl; ++k) order[k] = k;
      std::sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
        return tree.node(ln[a].node).depth > tree.node(ln[b].node).depth;
      });
      for (int32_t k : order) {
        for (int32_t h : ln[k].handles) ln[k].qcount += qn[h];
        if (ln[k].parent >= 0) ln[ln[k].parent].qcount += ln[k].qcount;
      }
    }
    // DFS preorder
    {
      int32_t pre = 0;
      std::vector<int32_t> st;
      for (size_t r = 0; r < roots.size(); ++r) {
        st.push_back(roots[r]);
        while (!st.empty()) {
          const int32_t k = st.back();
          st.pop_back();
          ln[k].pre = pre++;
          ln[k].root = static_cast<int32_t>(r);
          for (auto it = ln[k].children.rbegin(); it != ln[k].children.rend(); ++it) st.push_back(*it);
        }
      }
    }

    // 3. groups: subtrees with <= qg queries become units; units of one tree are
    //    packed in DFS order up to qg queries
    const int32_t rows = std::max(16, std::min<int32_t>(opt.max_rows, kMaxRows));
    const int32_t qg = std::max(1, std::min(kMaxGroupQueries, rows / q_per_kv));
    auto queries_of_handle = [&](int32_t h, std::vector<Query>& dst) {
      for (int32_t k = 0; k < qn[h]; ++k)
        dst.push_back({h, qbase[h] + k, static_cast<int32_t>(len[h] - qn[h] + k)});
    };
    std::vector<std::vector<Query>> group_q;
    std::vector<int32_t> group_root;
    {
      std::vector<int32_t> st, sub;
      for (size_t r = 0; r < roots.size(); ++r) {
        std::vector<std::vector<Query>> units;
        st.push_back(roots[r]);
        while (!st.empty()) {
          const int32_t k = st.back();
          st.pop_back();
          if (ln[k].qcount <= qg) {
            std::vector<Query> u;
            sub.push_back(k);
            while (!sub.empty()) {
              const int32_t s = sub.back();
              sub.pop_back();
              for (int32_t h : ln[s].handles) queries_of_handle(h, u);
              for (auto it = ln[s].children.rbegin(); it != ln[s].children.rend(); ++it) sub.push_back(*it);
            }
            if (!u.empty()) units.push_back(std::move(u));
          } else {
            std::vector<Query> own;
            for (int32_t h : ln[k].handles) queries_of_handle(h, own);
            for (size_t a = 0; a < own.size(); a += qg)
              units.emplace_back(own.begin() + a, own.begin() + std::min(own.size(), a + qg));
            for (auto it = ln[k].children.rbegin(); it != ln[k].children.rend(); ++it) st.push_back(*it);
          }
        }
        std::vector<Query> cur;
        for (auto& u : units) {
          if (!cur.empty() && cur.size() + u.size() > (size_t)qg) {
            group_q.push_back(std::move(cur));
            group_root.push_back(static_cast<int32_t>(r));
            cur.clear();
          }
          cur.insert(cur.end(), u.begin(), u.end());
        }
        if (!cur.empty()) {
          group_q.push_back(std::move(cur));
          group_root.push_back(static_cast<int32_t>(r));
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
    Plan& P = *out;
    P = Plan();
    P.nqueries = static_cast<int32_t>(total_q);
    P.causal = nq != nullptr;
    struct GroupOut {
      int32_t blk_begin, blk_count, root;
      bool partials;  // its queries have records in another group too
    };
    std::vector<GroupOut> gout;
    std::vector<std::vector<std::pair<int32_t, int32_t>>> qmem(total_q);  // (group, j)
    std::vector<uint64_t> mask(nl, 0);
    std::vector<int32_t> touched;
    const int32_t sub = std::max(1, 16 / q_per_kv);  // queries of a one-tile subgroup
    auto emit_group = [&](const Query* qs, int32_t n, int32_t root, bool partials) {
      const int32_t gi = static_cast<int32_t>(P.groups.size());
      DevGroup g;
      g.q_begin = static_cast<int32_t>(P.gq.size());
      g.nq = n;
      g.min_pos = INT32_MAX;
      g.pad1 = 0;
      for (int32_t j = 0; j < n; ++j) {
        P.gq.push_back(qs[j].global);
        P.gqpos.push_back(qs[j].pos);
        g.min_pos = std::min(g.min_pos, qs[j].pos);
        qmem[qs[j].global].push_back({gi, j});
      }
      P.groups.push_back(g);
      gout.push_back({static_cast<int32_t>(P.blocks.size()), 0, root, partials});
      return gi;
    };
    auto emit_node = [&](int32_t k, uint64_t m) {
      const Node& nd = tree.node(ln[k].node);
      const int32_t nb = static_cast<int32_t>(nd.blocks.size());
      for (int32_t b = 0; b < nb; ++b) {
        DevBlock e;
        e.id = nd.blocks[b];
        e.pos = static_cast<int32_t>(nd.base + 16 * (int64_t)b);
        e.valid = (b == nb - 1) ? nd.tail_valid() : 16;
        e.pad = 0;
        e.mask = m;
        P.blocks.push_back(e);
      }
    };
    auto close_group = [&]() { gout.back().blk_count = static_cast<int32_t>(P.blocks.size()) - gout.back().blk_begin; };
    // the subgroup a node's queries fit in, or -1
    auto narrow = [&](uint64_t m) {
      const int32_t lo = __builtin_ctzll(m), hi = 63 - __builtin_clzll(m);
      return lo / sub == hi / sub ? lo / sub : -1;
    };
    for (size_t g0 = 0; g0 < group_q.size(); ++g0) {
      const auto& qs = group_q[g0];
      const int32_t n = static_cast<int32_t>(qs.size());
      touched.clear();
      for (int32_t j = 0; j < n; ++j)
        for (int32_t k = loc[tip[qs[j].handle]]; k >= 0; k = ln[k].parent) {
          if (!mask[k]) touched.push_back(k);
          mask[k] |= 1ull << j;
        }
      std::sort(touched.begin(), touched.end(), [&](int32_t a, int32_t b) { return ln[a].pre < ln[b].pre; });
      bool cascade = false;
      if (opt.cascade && (n * q_per_kv + 15) / 16 >= 8 && n > sub) {
        int64_t all = 0, thin = 0;
        for (int32_t k : touched) {
          const int64_t nb = static_cast<int64_t>(tree.node(ln[k].node).blocks.size());
          all += nb;
          if (narrow(mask[k]) >= 0) thin += nb;
        }
        cascade = thin * 8 >= all && thin > 0;
      }
      emit_group(qs.data(), n, group_root[g0], cascade);
      for (int32_t k : touched)
        if (!cascade || narrow(mask[k]) < 0) emit_node(k, mask[k]);
      close_group();
      if (cascade) {
        for (int32_t t = 0; t * sub < n; ++t) {
          bool any = false;
          for (int32_t k : touched) any |= narrow(mask[k]) == t;
          if (!any) continue;
          emit_group(qs.data() + t * sub, std::min(sub, n - t * sub), group_root[g0], true);
          for (int32_t k : touched)
            if (narrow(mask[k]) == t) emit_node(k, mask[k] >> (t * sub));
          close_group();
        }
      }
      for (int32_t k : touched) mask[k] = 0;
    }
    const int32_t ngroups = static_cast<int32_t>(P.groups.size());

    // 5. split-K chunking and items.  The kernel classes of a call do not
    //    share the GPU well (a class's workgroups take whole CUs' registers or
    //    LDS, and side-stream joins cost more than the overlap gains), so each
    //    class is cut to fill the GPU on its own: about target_wgs / Hkv items,
    //    shared among its groups in proportion to their blocks, rounded down
    //    so that one round of workgroups holds them all.  A chunk stays long
    //    next to its partial record: at least min_chunk blocks for the
    //    register-tile classes, whose time is their memory time, and a quarter
    //    of that for the LDS-staged classes (3+ row tiles), whose time per
    //    block is several times longer; and at most kRowsMaxItemBlocks.
    //    An LDS-staged class whose work (blocks x row tiles) is smaller than
    //    that of the largest LDS-staged class present runs in that class's
    //    kernel instead (its extra waves idle): one launch and one ramp fewer.
    std::vector<int8_t> gclass(ngroups);
    int64_t class_work[kKernelClasses] = {0, 0, 0, 0, 0, 0};
    for (int32_t gi = 0; gi < ngroups; ++gi) {
      const int32_t tiles = (P.groups[gi].nq * q_per_kv + 15) / 16;
      gclass[gi] = static_cast<int8_t>(kernel_class(tiles));
      class_work[gclass[gi]] += static_cast<int64_t>(gout[gi].blk_count) * tiles;
    }
    int top = -1;
    for (int c = 2; c < kKernelClasses; ++c)
      if (class_work[c] > 0) top = c;
    if (top > 2)
      for (int32_t gi = 0; gi < ngroups; ++gi)
        if (gclass[gi] >= 2 && gclass[gi] < top && class_work[gclass[gi]] < class_work[top]) gclass[gi] = top;
    int64_t class_blocks[kKernelClasses] = {0, 0, 0, 0, 0, 0};
    auto class_of = [&](int32_t gi) { return static_cast<int>(gclass[gi]); };
    for (int32_t gi = 0; gi < ngroups; ++gi) class_blocks[class_of(gi)] += gout[gi].blk_count;
    const int64_t class_items = std::max<int64_t>(1, std::max<int32_t>(1, opt.target_wgs) / num_kv_heads);
    auto chunks_of = [&](int32_t gi) -> int32_t {
      const int cls = class_of(gi);
      const int64_t nb = gout[gi].blk_count;
      const int64_t floor = std::max<int32_t>(1, cls < 2 ? opt.min_chunk : opt.min_chunk / 4);
      // the 4- and 8-tile LDS-staged shapes fit two workgroups per CU, and
      // two per CU stream faster than one with a deeper ring: twice the items
      const int64_t want = (cls == 2 || cls == 4) ? 2 * class_items : class_items;
      int64_t nc = nb * want / class_blocks[cls];
      nc = std::min(nc, nb / floor);
      nc = std::max<int64_t>(nc, (nb + kRowsMaxItemBlocks - 1) / kRowsMaxItemBlocks);
      return static_cast<int32_t>(std::max<int64_t>(nc, 1));
    };
    struct Tmp {
      DevItem it;
      int32_t tiles, root, chunk;
    };
    std::vector<Tmp> tmp;
    int64_t slots = 0;
    for (int32_t gi = 0; gi < ngroups; ++gi) {
      const int32_t nb = gout[gi].blk_count;
      if (nb == 0) continue;
      const int32_t nc = chunks_of(gi);
      const int32_t tiles = class_of(gi);
      int32_t at = 0;
      for (int32_t c = 0; c < nc; ++c) {
        const int32_t cnt = nb / nc + (c < nb % nc ? 1 : 0);
        Tmp t;
        t.it.group = gi;
        t.it.blk_begin = gout[gi].blk_begin + at;
        t.it.blk_count = cnt;
        t.it.q_begin = P.groups[gi].q_begin;
        t.it.nq = P.groups[gi].nq;
        t.it.min_pos = P.groups[gi].min_pos;
        t.it.pad = 0;
        if (nc == 1 && !gout[gi].partials) {
          t.it.part_base = -1;
        } else {
          t.it.part_base = static_cast<int32_t>(slots);
          slots += static_cast<int64_t>(P.groups[gi].nq) * q_per_kv * num_kv_heads;
          if (slots > INT32_MAX) return TKV_E_RANGE;
        }
        t.tiles = tiles;
        t.root = gout[gi].root;
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
    // items share L2
    std::stable_sort(tmp.begin(), tmp.end(), [](const Tmp& a, const Tmp& b) {
      if (a.tiles != b.tiles) return a.tiles < b.tiles;
      if (a.it.blk_count != b.it.blk_count) return a.it.blk_count > b.it.blk_count;
      if (a.root != b.root) return a.root < b.root;
      if (a.chunk != b.chunk) return a.chunk < b.chunk;
      return a.it.group < b.it.group;
    });
    P.items.resize(tmp.size());
    for (int t = 0; t <= kKernelClasses; ++t) P.bucket_begin[t] = 0;
    std::vector<std::vector<int32_t>> gitems(ngroups);
    for (size_t k = 0; k < tmp.size(); ++k) {
      P.items[k] = tmp[k].it;
      gitems[tmp[k].it.group].push_back(static_cast<int32_t>(k));
    }
    for (int c = 0; c < kKernelClasses; ++c) {
      int32_t cnt = 0;
      for (const auto& x : tmp) cnt += (x.tiles <= c);
      P.bucket_begin[c + 1] = cnt;
      P.bucket_max_blocks[c] = 0;
      P.bucket_blocks[c] = 0;
    }
    for (const auto& x : tmp) {
      P.bucket_max_blocks[x.tiles] = std::max(P.bucket_max_blocks[x.tiles], x.it.blk_count);
      P.bucket_blocks[x.tiles] += x.it.blk_count;
    }
    // merge records: every partial of a query, in the order its groups were made
    P.merge.resize(total_q);
    for (int64_t q = 0; q < total_q; ++q) {
      DevMerge m;
      m.p_begin = static_cast<int32_t>(P.parts.size());
      int32_t direct = 0;
      for (const auto& gj : qmem[q])
        for (int32_t item : gitems[gj.first]) {
          if (P.items[item].part_base < 0) {
            ++direct;
            continue;
          }
          P.parts.push_back({P.items[item].part_base + gj.second * q_per_kv * num_kv_heads, item});
        }
      m.p_count = static_cast<int32_t>(P.parts.size()) - m.p_begin;
      if (direct + m.p_count == 0 || (direct > 0 && (direct > 1 || m.p_count > 0))) return TKV_E_INVAL;
      P.merge[q] = m;
      if (m.p_count) P.any_merge = true;
    }

    // statistics: distinct blocks read and their valid slots
    {
      std::vector<std::pair<int32_t, int32_t>> ids;
      ids.reserve(P.blocks.size());
      for (const auto& b : P.blocks) ids.push_back({b.id, b.valid});
      std::sort(ids.begin(), ids.end());
      ids.erase(std::unique(ids.begin(), ids.end(),
                            [](const auto& a, const auto& b) { return a.first == b.first; }),
                ids.end());
      P.unique_blocks = static_cast<int32_t>(ids.size());
      for (const auto& x : ids) P.unique_tokens += x.second;
    }
    P.layout();
  } catch (const std::bad_alloc&) {
    return TKV_E_NOMEM;
  }
  return TKV_OK;
}

}  // namespace tkv
