// Host check of what the planner's output means, run by tests/test_host_core.py
// (also under AddressSanitizer and UndefinedBehaviorSanitizer).  For seeded
// random sessions of forks, appends, truncations and releases, and planner
// options drawn per session (row limit 16..256, one-tile subgroups on or off,
// 1..16 query heads per KV head, chunk floors and workgroup targets), the plan
// of a decode or verify batch must satisfy, from the tree alone:
//   1. every query sees exactly the (block, slot) pairs of its own path up to
//      its position, each once, summed over all the items of all its groups
//      (block visibility masks, valid counts, the causal limit);
//   2. each group's items cover its block list exactly, in order, with the
//      group's queries, position minimum and the list's tail blocks;
//   3. a query's output is written directly by exactly one item or assembled
//      by the merge from one partial record per item of its groups that holds
//      a block the query sees (the item's query mask), at the slot that item
//      writes for it, and no two records share a slot;
//   4. the serialised layout's sections are disjoint, aligned and inside the
//      buffer, and kernel classes and their longest items agree with the items.
// Prints one line per session and exits non-zero on the first violation.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <set>
#include <utility>
#include <vector>

#include "plan.h"
#include "tree.h"

using namespace tkv;

namespace {

uint64_t mix(uint64_t x) {  // SplitMix64 finaliser
  x += 0x9e3779b97f4a7c15ull;
  x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
  x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
  return x ^ (x >> 31);
}

struct Rng {
  uint64_t s;
  int32_t below(int32_t n) { return static_cast<int32_t>(mix(s++) % static_cast<uint64_t>(n)); }
};

int fail(int sess, const char* what) {
  std::printf("session %d: %s\n", sess, what);
  return 1;
}

}  // namespace

int main(int argc, char** argv) {
  const int sessions = argc > 1 ? atoi(argv[1]) : 100;
  int64_t queries_checked = 0, pairs_checked = 0;
  for (int sess = 0; sess < sessions; ++sess) {
    Rng r{0xc0ffee00ull + static_cast<uint64_t>(sess) * 104729};
    Tree t(6000);
    std::vector<tkv_seq> live;
    tkv_seq root;
    t.seq_new(&root);
    live.push_back(root);
    Placement pl;
    const int steps = 40 + r.below(160);
    for (int step = 0; step < steps; ++step) {
      const int32_t c = r.below(10);
      const size_t hi = static_cast<size_t>(r.below(static_cast<int32_t>(live.size())));
      if (c < 5) {
        t.append(live[hi], 1 + r.below(r.below(4) == 0 ? 300 : 40), &pl);
      } else if (c < 7 && live.size() < 70) {
        const int32_t n = 1 + r.below(5);
        std::vector<tkv_seq> kids(n);
        if (t.fork(live[hi], n, kids.data()) == TKV_OK) live.insert(live.end(), kids.begin(), kids.end());
      } else if (c < 8) {
        int64_t len;
        t.seq_len(live[hi], &len);
        t.truncate(live[hi], len - r.below(20));  // may be refused (shared)
      } else if (live.size() > 3) {
        t.release(live[hi]);
        live.erase(live.begin() + hi);
      }
    }
    const bool verify = sess % 2 == 1;
    std::vector<tkv_seq> seqs;
    std::vector<int32_t> nq;
    for (tkv_seq h : live) {
      int64_t len;
      t.seq_len(h, &len);
      if (len == 0 || r.below(4) == 0) continue;
      seqs.push_back(h);
      if (r.below(5) == 0) seqs.push_back(h);  // a handle may appear twice
      nq.push_back(1 + r.below(static_cast<int32_t>(len < 12 ? len : 12)));
      if (seqs.size() > nq.size()) nq.push_back(nq.back());
    }
    if (seqs.empty()) continue;
    static const int32_t kQpk[] = {1, 2, 4, 8, 16};
    static const int32_t kRows[] = {16, 32, 64, 128, 256};
    const int32_t qpk = kQpk[r.below(5)];
    const int32_t hkv = 1 + r.below(3);
    PlanOptions opt;
    opt.max_rows = kRows[r.below(5)];
    opt.cascade = r.below(2);
    opt.min_chunk = 1 + r.below(40);
    opt.target_wgs = 1 + r.below(800);
    opt.two_per_cu = r.below(2);
    const int32_t* nqp = verify ? nq.data() : nullptr;
    const int32_t nseq = static_cast<int32_t>(seqs.size());
    PlanScratch scratch;
    Plan P;
    if (build_plan(t, seqs.data(), nqp, nseq, qpk, hkv, opt, &P, &scratch)) return fail(sess, "build failed");

    // the expected view of every query: its handle's path (block, slot) pairs up to its position
    std::vector<int32_t> qh, qpos;  // handle (batch index) and position per global query
    for (int32_t i = 0; i < nseq; ++i) {
      int64_t len;
      t.seq_len(seqs[i], &len);
      const int32_t m = verify ? nq[i] : 1;
      for (int32_t k = 0; k < m; ++k) {
        qh.push_back(i);
        qpos.push_back(static_cast<int32_t>(len - m + k));
      }
    }
    const int32_t nqt = static_cast<int32_t>(qh.size());
    if (P.nqueries != nqt) return fail(sess, "query count");

    // 4. layout
    {
      const size_t offs[] = {P.off_items, P.off_gq, P.off_gqpos, P.off_blocks, P.off_parts, P.off_merge, P.bytes};
      const size_t sizes[] = {P.items.size() * sizeof(DevItem), P.gq.size() * 4, P.gqpos.size() * 4,
                              P.blocks.size() * sizeof(DevBlock), P.parts.size() * sizeof(DevPart),
                              P.merge.size() * sizeof(DevMerge)};
      for (int k = 0; k < 6; ++k) {
        if (offs[k] % 256 != 0) return fail(sess, "section not 256-byte aligned");
        if (offs[k] + sizes[k] > offs[k + 1]) return fail(sess, "sections overlap");
      }
      int32_t begin = 0;
      for (int cls = 0; cls < kKernelClasses; ++cls) {
        if (P.bucket_begin[cls] != begin) return fail(sess, "class buckets not contiguous");
        int32_t longest = 0;
        for (int32_t k = P.bucket_begin[cls]; k < P.bucket_begin[cls + 1]; ++k)
          longest = std::max(longest, P.items[k].blk_count);
        if (longest != P.bucket_max_blocks[cls]) return fail(sess, "class longest item");
        begin = P.bucket_begin[cls + 1];
      }
      if (begin != static_cast<int32_t>(P.items.size())) return fail(sess, "classes do not cover the items");
    }

    // 2. items cover each group's list exactly
    const int32_t ng = static_cast<int32_t>(P.groups.size());
    std::vector<std::vector<int32_t>> items_of(ng);
    for (int32_t k = 0; k < static_cast<int32_t>(P.items.size()); ++k) {
      const DevItem& it = P.items[k];
      if (it.group < 0 || it.group >= ng) return fail(sess, "item group");
      const DevGroup& g = P.groups[it.group];
      if (it.q_begin != g.q_begin || it.nq != g.nq || it.min_pos != g.min_pos) return fail(sess, "item group fields");
      if (it.blk_count < 1 || it.blk_begin < 0 || it.blk_begin + it.blk_count > static_cast<int32_t>(P.blocks.size()))
        return fail(sess, "item block range");
      if (it.blk_count > kRowsMaxItemBlocks) return fail(sess, "item longer than a staged list");
      items_of[it.group].push_back(k);
      // tail blocks of the item
      int32_t lo = -1, cnt = 0;
      for (size_t ti = 0; ti < P.tail_entry.size(); ++ti)
        if (P.tail_entry[ti] >= it.blk_begin && P.tail_entry[ti] < it.blk_begin + it.blk_count) {
          if (lo < 0) lo = static_cast<int32_t>(ti);
          ++cnt;
        }
      const int32_t want = cnt > 0 ? (lo | (cnt << 16)) : 0;
      if (it.tails != want) return fail(sess, "item tail range");
    }
    for (int32_t g = 0; g < ng; ++g) {
      auto& v = items_of[g];
      std::sort(v.begin(), v.end(), [&](int32_t a, int32_t b) { return P.items[a].blk_begin < P.items[b].blk_begin; });
      for (size_t k = 1; k < v.size(); ++k)
        if (P.items[v[k]].blk_begin != P.items[v[k - 1]].blk_begin + P.items[v[k - 1]].blk_count)
          return fail(sess, "items of a group leave a gap or overlap");
      const DevGroup& gr = P.groups[g];
      if (gr.nq < 1 || gr.nq > kMaxGroupQueries || gr.nq * qpk > kMaxRows) return fail(sess, "group size");
      int32_t mn = INT32_MAX;
      for (int32_t j = 0; j < gr.nq; ++j) {
        const int32_t q = P.gq[gr.q_begin + j];
        if (q < 0 || q >= nqt) return fail(sess, "group query index");
        if (P.gqpos[gr.q_begin + j] != qpos[q]) return fail(sess, "query position");
        mn = std::min(mn, qpos[q]);
      }
      if (mn != gr.min_pos) return fail(sess, "group position minimum");
    }

    // 1 and 3: per query, what its groups' items show it, and where its records go
    std::vector<std::vector<std::pair<int32_t, int32_t>>> seen(nqt);  // (group, index in group)
    for (int32_t g = 0; g < ng; ++g)
      for (int32_t j = 0; j < P.groups[g].nq; ++j) seen[P.gq[P.groups[g].q_begin + j]].push_back({g, j});
    std::set<int64_t> slots_used;
    for (int32_t q = 0; q < nqt; ++q) {
      if (seen[q].empty() || seen[q].size() > 2) return fail(sess, "a query in no group or in more than two");
      std::map<std::pair<int32_t, int32_t>, int32_t> count;  // (block id, slot) -> times seen
      std::set<int32_t> expected_slots;
      int32_t direct = 0, partial = 0;
      for (auto [g, j] : seen[q]) {
        for (int32_t k : items_of[g]) {
          const DevItem& it = P.items[k];
          uint64_t om = 0;
          for (int32_t b = it.blk_begin; b < it.blk_begin + it.blk_count; ++b) om |= P.blocks[b].mask;
          if (om != it.qmask) return fail(sess, "item query mask is not the OR of its blocks' masks");
          if (it.part_base < 0) ++direct;
          else if ((it.qmask >> j) & 1ull) {
            ++partial;
            const int64_t slot0 = static_cast<int64_t>(it.part_base) + static_cast<int64_t>(j) * qpk * hkv;
            expected_slots.insert(static_cast<int32_t>(slot0));
          }
          for (int32_t b = it.blk_begin; b < it.blk_begin + it.blk_count; ++b) {
            const DevBlock& e = P.blocks[b];
            if (!((e.mask >> j) & 1ull)) continue;
            for (int32_t s = 0; s < e.valid; ++s) {
              if (verify && e.pos + s > qpos[q]) continue;
              ++count[{e.id, s}];
            }
          }
        }
      }
      // expected: the handle's table, positions 0 .. qpos
      std::vector<int32_t> ids(8192), valid(8192);
      int32_t n = 0;
      if (t.block_table(seqs[qh[q]], ids.data(), valid.data(), 8192, &n)) return fail(sess, "table");
      std::map<std::pair<int32_t, int32_t>, int32_t> want;
      int32_t pos = 0;
      for (int32_t b = 0; b < n; ++b)
        for (int32_t s = 0; s < valid[b]; ++s, ++pos)
          if (pos <= qpos[q]) want[{ids[b], s}] = 1;
      if (count != want) return fail(sess, "a query does not see exactly its path once");
      pairs_checked += static_cast<int64_t>(want.size());
      const DevMerge& m = P.merge[q];
      if (direct + partial == 0) return fail(sess, "a query with no item");
      if (direct > 0 && (direct > 1 || partial > 0)) return fail(sess, "direct output mixed with records");
      if (m.p_count != partial) return fail(sess, "merge record count");
      std::set<int32_t> got;
      for (int32_t p = m.p_begin; p < m.p_begin + m.p_count; ++p) {
        got.insert(P.parts[p].slot0);
        if (P.parts[p].slot0 < 0 || static_cast<int64_t>(P.parts[p].slot0) + qpk * hkv > P.partial_slots)
          return fail(sess, "record slot outside the workspace");
        for (int32_t h = 0; h < qpk * hkv; ++h)
          if (!slots_used.insert(static_cast<int64_t>(P.parts[p].slot0) + h).second)
            return fail(sess, "two records share a slot");
      }
      if (got != expected_slots) return fail(sess, "merge records do not match the items' slots");
      ++queries_checked;
    }
    std::printf("session %d %s: %d handles, %d queries, %d groups, %zu items, qpk %d, rows %d, cascade %d ok\n", sess,
                verify ? "verify" : "decode", nseq, nqt, ng, P.items.size(), qpk, opt.max_rows, opt.cascade);
  }
  std::printf("all sessions ok: %lld queries, %lld (block, slot) pairs\n", static_cast<long long>(queries_checked),
              static_cast<long long>(pairs_checked));
  return 0;
}
