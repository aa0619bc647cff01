// Host check of the planner's in-place update (patch_plan), run by
// tests/test_host_core.py (also under AddressSanitizer and
// UndefinedBehaviorSanitizer): for seeded random sessions of forks, appends,
// truncations and releases, and planner options drawn per session (row limit
// 16..256, one-tile subgroups on or off, 1..16 query heads per KV head, chunk
// floors and workgroup targets), build the plan of a decode or verify batch, then
// repeatedly append tokens that fit in tip nodes' last blocks, patch the plan,
// and require (1) the patched plan to equal a fresh build byte for byte and
// (2) the changed words, written over the previous serialisation, to give the
// same bytes (what the device copy receives).  Prints one line per session and
// exits non-zero on the first mismatch.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
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

std::vector<char> bytes_of(const Plan& p) {
  std::vector<char> b(p.bytes);
  p.serialise(b.data());
  return b;
}

bool same(const Plan& a, const Plan& b) {
  if (a.bytes != b.bytes || a.unique_blocks != b.unique_blocks || a.unique_tokens != b.unique_tokens) return false;
  if (a.groups.size() != b.groups.size()) return false;
  for (size_t g = 0; g < a.groups.size(); ++g)
    if (a.groups[g].min_pos != b.groups[g].min_pos || a.groups[g].nq != b.groups[g].nq) return false;
  return bytes_of(a) == bytes_of(b);
}

}  // namespace

int main(int argc, char** argv) {
  const int sessions = argc > 1 ? atoi(argv[1]) : 40;
  int64_t patched_words = 0, rounds = 0;
  for (int sess = 0; sess < sessions; ++sess) {
    Rng r{0x5eed0000ull + static_cast<uint64_t>(sess) * 7919};
    Tree t(4000);
    std::vector<tkv_seq> live;
    tkv_seq root;
    t.seq_new(&root);
    live.push_back(root);
    Placement pl;
    for (int step = 0; step < 150; ++step) {
      const int32_t c = r.below(10);
      const size_t hi = static_cast<size_t>(r.below(static_cast<int32_t>(live.size())));
      if (c < 5) {
        t.append(live[hi], 1 + r.below(60), &pl);
      } else if (c < 7 && live.size() < 40) {
        const int32_t n = 1 + r.below(4);
        std::vector<tkv_seq> kids(n);
        if (t.fork(live[hi], n, kids.data()) == TKV_OK) live.insert(live.end(), kids.begin(), kids.end());
      } else if (c < 8) {
        int64_t len;
        t.seq_len(live[hi], &len);
        t.truncate(live[hi], len - r.below(20));  // may be refused (shared), which is fine
      } else if (live.size() > 3) {
        t.release(live[hi]);
        live.erase(live.begin() + hi);
      }
    }
    // the batch: every non-empty handle (decode), or about half of them with
    // query counts (verify)
    const bool verify = sess % 2 == 1;
    std::vector<tkv_seq> seqs;
    std::vector<int32_t> nq;
    for (tkv_seq h : live) {
      int64_t len;
      t.seq_len(h, &len);
      if (len == 0 || (verify && r.below(2))) continue;
      seqs.push_back(h);
      nq.push_back(1 + r.below(static_cast<int32_t>(len < 12 ? len : 12)));
    }
    if (seqs.empty()) continue;
    static const int32_t kQpk[] = {1, 2, 4, 8, 16};
    static const int32_t kRows[] = {16, 32, 64, 128, 256};
    const int32_t qpk = kQpk[r.below(5)], hkv = 2;
    PlanOptions opt;
    opt.min_chunk = 1 + r.below(32);
    opt.target_wgs = 2 + r.below(600);
    opt.max_rows = kRows[r.below(5)];
    opt.cascade = r.below(2);
    PlanScratch scratch;
    Plan live_plan, fresh;
    const int32_t* nqp = verify ? nq.data() : nullptr;
    if (build_plan(t, seqs.data(), nqp, static_cast<int32_t>(seqs.size()), qpk, hkv, opt, &live_plan, &scratch)) {
      std::printf("session %d: build failed\n", sess);
      return 1;
    }
    for (int round = 0; round < 12; ++round) {
      const uint64_t shape = t.shape_epoch();
      // appends that fit in the tip's last block (unfrozen tips with room)
      for (size_t i = 0; i < seqs.size(); ++i) {
        if (r.below(3) == 0) continue;
        int32_t tip;
        if (t.resolve(seqs[i], &tip)) continue;
        const Node& nd = t.node(tip);
        if (nd.frozen || nd.blocks.empty()) continue;  // the append would start a node or a block
        const int32_t room = 16 - nd.tail_valid();
        if (room == 0) continue;
        t.append(seqs[i], 1 + r.below(room), &pl);
      }
      if (t.shape_epoch() != shape) {
        std::printf("session %d: an in-block append changed the shape epoch\n", sess);
        return 1;
      }
      std::vector<char> before = bytes_of(live_plan);
      std::vector<PlanWord> words;
      patch_plan(t, &live_plan, &words);
      if (build_plan(t, seqs.data(), nqp, static_cast<int32_t>(seqs.size()), qpk, hkv, opt, &fresh, &scratch)) {
        std::printf("session %d: rebuild failed\n", sess);
        return 1;
      }
      if (!same(live_plan, fresh)) {
        std::printf("session %d round %d: patched plan differs from a fresh build\n", sess, round);
        return 1;
      }
      for (const PlanWord& w : words) {
        if (static_cast<size_t>(w.word) * 4 + 4 > before.size()) {
          std::printf("session %d: changed word %u outside the plan\n", sess, w.word);
          return 1;
        }
        std::memcpy(before.data() + static_cast<size_t>(w.word) * 4, &w.value, 4);
      }
      if (before != bytes_of(fresh)) {
        std::printf("session %d round %d: changed words do not reproduce the fresh bytes\n", sess, round);
        return 1;
      }
      patched_words += static_cast<int64_t>(words.size());
      ++rounds;
    }
    std::printf("session %d %s: %zu handles, %zu block entries, %zu tails ok\n", sess, verify ? "verify" : "decode",
                seqs.size(), live_plan.blocks.size(), live_plan.tail_entry.size());
  }
  std::printf("all sessions ok: %lld rounds, %lld changed words\n", static_cast<long long>(rounds),
              static_cast<long long>(patched_words));
  return 0;
}
