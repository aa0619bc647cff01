// Fork latency of libtkv.so, host side only (no device memory is touched).
//
// For each prefix length P (tokens) and path depth D (nodes on the parent's
// root-to-tip path), a handle is built with D nodes holding P tokens in
// total, then tkv_fork(parent, n) is timed for n in {1, 4, 16}: batches of 64
// forks are timed as a whole (their children released untimed after each
// batch), and the median over batches of the per-fork time is printed.  The
// claim checked is the one of the Dendrite article ("technical deep dive") and
// demo tape ("Fork benchmark results"): fork cost does not grow with the
// prefix, and here not with depth either.
//
// Output: one JSON object {"P:D:n": ns, ...} on stdout.
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <chrono>
#include <string>
#include <vector>

#include "tkv.h"

namespace {

int check(int rc, const char* what) {
  if (rc != TKV_OK) {
    fprintf(stderr, "%s failed: %s\n", what, tkv_strerror(rc));
    exit(1);
  }
  return rc;
}

double median_fork_ns(int64_t prefix, int depth, int n, int batches) {
  tkv_config cfg{};
  cfg.num_layers = 1;
  cfg.num_q_heads = 32;
  cfg.num_kv_heads = 8;
  cfg.head_dim = 128;
  cfg.block_size = 16;
  cfg.num_blocks = static_cast<int32_t>(prefix / 16 + depth + 64);
  cfg.dtype = TKV_BF16;
  tkv_cache* c = nullptr;
  check(tkv_create(&cfg, &c), "tkv_create");
  tkv_seq s = 0;
  check(tkv_seq_new(c, &s), "tkv_seq_new");
  // D nodes: append a share of the prefix, then fork once to freeze the tip
  int64_t left = prefix;
  for (int i = 0; i < depth; ++i) {
    const int64_t take = std::max<int64_t>(1, left / (depth - i));
    check(tkv_append(c, s, static_cast<int32_t>(take), nullptr, nullptr, nullptr), "tkv_append");
    left -= take;
    if (i + 1 < depth) {
      tkv_seq child = 0;
      check(tkv_fork(c, s, 1, &child), "tkv_fork");
      check(tkv_release(c, s), "tkv_release");
      s = child;
    }
  }
  constexpr int kPerBatch = 64;
  std::vector<tkv_seq> kids(static_cast<size_t>(kPerBatch) * n);
  std::vector<double> per_fork;
  for (int b = 0; b < batches + 5; ++b) {
    const auto t0 = std::chrono::steady_clock::now();
    for (int k = 0; k < kPerBatch; ++k) check(tkv_fork(c, s, n, &kids[static_cast<size_t>(k) * n]), "tkv_fork");
    const auto t1 = std::chrono::steady_clock::now();
    for (auto h : kids) check(tkv_release(c, h), "tkv_release");
    if (b >= 5) per_fork.push_back(std::chrono::duration<double, std::nano>(t1 - t0).count() / kPerBatch);
  }
  check(tkv_release(c, s), "tkv_release");
  check(tkv_destroy(c), "tkv_destroy");
  std::sort(per_fork.begin(), per_fork.end());
  return per_fork[per_fork.size() / 2];
}

}  // namespace

int main(int argc, char** argv) {
  const int batches = argc > 1 ? atoi(argv[1]) : 400;
  const int64_t prefixes[] = {16, 256, 4096, 65536};
  const int depths[] = {1, 10, 50, 100, 500};
  const int ns[] = {1, 4, 16};
  std::string out = "{";
  bool first = true;
  for (int64_t p : prefixes)
    for (int d : depths) {
      if (d > p) continue;  // every node holds at least one token
      for (int n : ns) {
        char buf[96];
        snprintf(buf, sizeof buf, "%s\"%lld:%d:%d\": %.1f", first ? "" : ", ", static_cast<long long>(p), d, n,
                 median_fork_ns(p, d, n, batches));
        out += buf;
        first = false;
      }
    }
  out += "}";
  puts(out.c_str());
  return 0;
}
