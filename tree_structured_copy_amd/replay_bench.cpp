// Native replay of a workload recipe through libtkv.so: time and memory of the
// loops whose host calls are too many and too cheap to drive from Python
// (ctypes costs about a microsecond per call).  They are the speculative loop
// (fork, draft, verify, accept or roll back: the DSpark blog's second layer,
// the Dendrite article's multi-draft speculation) and the tree-search
// simulations of the Dendrite demo tape.
//
// Input: a file holding workloads.recipes.ops_text of the recipe.  The recipe
// runs three times on one cache; between the passes every live handle is
// released, which leaves the cache empty but keeps what a long-running caller
// would hold (plan buffers, pinned staging).  The first pass sizes the
// workspace and warms the GPU.  The second is timed from its time_begin line
// to the end, synchronised on both sides.  The third repeats it with the
// library's profiling events on, for the attention kernels' own time.  K, V
// and Q hold a constant fill: the parity tests replay the same recipes
// against the oracle.
//
// With --host the cache is host-only: appends reserve slots, attention calls
// have their plans built (the host work a loop needs per call) but are not
// run, and no HIP call is made (the block and fork figures still hold; wall_ms
// is then the loop's tree and planner time).
//
// Output: one JSON object on stdout with, for the measured part,
//   wall_ms         wall time;
//   attend_calls, decode_queries, verify_tokens;
//   attend_kernel_ms  the attention kernels' time (partial + merge, HIP events
//                     the library records on the stream);
//   forks, fork_ns    calls and mean host time of tkv_fork;
//   appended_tokens;
//   peak_blocks, cow_peak_bytes   most blocks in use at once, and their bytes
//                                 over all layers, K and V;
//   full_copy_bytes   what copying the parent's whole path at every fork would
//                     have allocated (the design the article compares with);
//   plans_built, plans_patched, plans_uploaded, plans_reused    from the counters.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <chrono>
#include <sstream>
#include <string>
#include <vector>

#include "tkv.h"

namespace {

void die(const char* what, const char* why) {
  fprintf(stderr, "replay_bench: %s: %s\n", what, why);
  exit(1);
}

void check(int rc, const char* what) {
  if (rc != TKV_OK) die(what, tkv_strerror(rc));
}

void hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) die(what, hipGetErrorString(e));
}

struct Op {
  std::string kind;
  std::vector<int64_t> a;  // the numbers after the kind, as written
};

struct Config {
  int32_t layers = 0, hq = 0, hkv = 0, d = 0, blocks = 0, bf16 = 1;
};

struct Stats {
  double wall_ms = 0, attend_ms = 0, merge_ms = 0, fork_ns = 0;
  int64_t attend_calls = 0, decode_queries = 0, verify_tokens = 0, forks = 0, appended = 0;
  int64_t peak_blocks = 0, full_copy_tokens = 0;
  tkv_counters counters{};
};

double now_ms() {
  return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now().time_since_epoch()).count();
}

class Replayer {
 public:
  Replayer(const Config& cfg, const std::vector<Op>& ops, bool host) : cfg_(cfg), ops_(ops), host_(host) {
    elem_ = cfg.bf16 ? 2 : 4;
    int64_t max_src = 1, max_rows = 1, max_name = 0;
    for (const Op& op : ops) {
      if (op.kind == "append") max_src = std::max(max_src, op.a[1]);
      if (op.kind == "append_batch" || op.kind == "reserve_batch") {
        int64_t t = 0;
        for (int64_t i = 0; i < op.a[0]; ++i) t += op.a[2 + 2 * i];
        max_src = std::max(max_src, t);
      }
      if (op.kind == "decode" || op.kind == "decode_new") max_rows = std::max(max_rows, op.a[1]);
      if (op.kind == "verify" || op.kind == "verify_new") {
        int64_t t = 0;
        for (int64_t i = 0; i < op.a[1]; ++i) t += op.a[3 + 2 * i];
        max_rows = std::max(max_rows, t);
      }
      for (int64_t x : op.a) max_name = std::max(max_name, x);
    }
    names_ = static_cast<size_t>(max_name) + 1;
    if (host_) return;
    const size_t pool = static_cast<size_t>(cfg.layers) * cfg.blocks * cfg.hkv * 16 * cfg.d * elem_;
    const size_t src = static_cast<size_t>(cfg.layers) * max_src * cfg.hkv * cfg.d * elem_;
    const size_t q = static_cast<size_t>(max_rows) * cfg.hq * cfg.d * elem_;
    const size_t out = static_cast<size_t>(max_rows) * cfg.hq * cfg.d * 4;
    hip_check(hipStreamCreateWithFlags(&stream_, hipStreamNonBlocking), "hipStreamCreate");
    for (auto [p, n] : {std::pair<void**, size_t>{&kpool_, pool}, {&vpool_, pool}, {&ksrc_, src}, {&vsrc_, src},
                        {&q_, q}, {&out_, out}}) {
      hip_check(hipMalloc(p, n), "hipMalloc");
      // about 0.0115 in bf16 and in fp32: finite inputs of no consequence for timing
      hip_check(hipMemsetAsync(*p, 0x3c, n, stream_), "hipMemsetAsync");
    }
    hip_check(hipStreamSynchronize(stream_), "hipStreamSynchronize");
  }

  ~Replayer() {
    if (cache_) (void)tkv_destroy(cache_);
    for (void* p : {kpool_, vpool_, ksrc_, vsrc_, q_, out_, ws_})
      if (p) (void)hipFree(p);
    if (stream_) (void)hipStreamDestroy(stream_);
  }

  void create() {
    tkv_config c{};
    c.num_layers = cfg_.layers;
    c.num_q_heads = cfg_.hq;
    c.num_kv_heads = cfg_.hkv;
    c.head_dim = cfg_.d;
    c.block_size = 16;
    c.num_blocks = cfg_.blocks;
    c.dtype = cfg_.bf16 ? TKV_BF16 : TKV_F32;
    c.k_pool = kpool_;  // both null with --host
    c.v_pool = vpool_;
    check(tkv_create(&c, &cache_), "tkv_create");
  }

  Stats run(bool measure) {
    if (!cache_) create();
    tkv_cache* cache = cache_;
    std::vector<tkv_seq> h(names_, 0);
    std::vector<tkv_seq> seqs;
    std::vector<int32_t> counts;
    Stats st;
    bool timed = false;
    double t0 = 0;
    tkv_counters base{};
    int32_t nfree = 0;
    auto sample_blocks = [&]() {
      check(tkv_num_free(cache, &nfree), "tkv_num_free");
      st.peak_blocks = std::max<int64_t>(st.peak_blocks, cfg_.blocks - nfree);
    };
    for (const Op& op : ops_) {
      const auto& a = op.a;
      if (op.kind == "time_begin") {
        sync();
        check(tkv_get_counters(cache, &base), "tkv_get_counters");
        if (measure && !host_) check(tkv_profile_enable(cache, 1), "tkv_profile_enable");
        timed = true;
        st = Stats();
        sample_blocks();
        t0 = now_ms();
      } else if (op.kind == "new") {
        check(tkv_seq_new(cache, &h[a[0]]), "tkv_seq_new");
      } else if (op.kind == "append") {
        check(tkv_append(cache, h[a[0]], static_cast<int32_t>(a[1]), ksrc_, vsrc_, stream_), "tkv_append");
        st.appended += a[1];
        sample_blocks();
      } else if (op.kind == "append_batch") {
        seqs.clear();
        counts.clear();
        for (int64_t i = 0; i < a[0]; ++i) {
          seqs.push_back(h[a[1 + 2 * i]]);
          counts.push_back(static_cast<int32_t>(a[2 + 2 * i]));
          st.appended += a[2 + 2 * i];
        }
        check(tkv_append_batch(cache, seqs.data(), counts.data(), static_cast<int32_t>(seqs.size()), ksrc_, vsrc_,
                               stream_),
              "tkv_append_batch");
        sample_blocks();
      } else if (op.kind == "reserve_batch") {
        // slots only: the decode_new call that follows writes their K/V
        seqs.clear();
        counts.clear();
        for (int64_t i = 0; i < a[0]; ++i) {
          seqs.push_back(h[a[1 + 2 * i]]);
          counts.push_back(static_cast<int32_t>(a[2 + 2 * i]));
          st.appended += a[2 + 2 * i];
        }
        check(tkv_append_batch(cache, seqs.data(), counts.data(), static_cast<int32_t>(seqs.size()), nullptr,
                               nullptr, stream_),
              "tkv_append_batch");
        sample_blocks();
      } else if (op.kind == "decode_new") {
        seqs.clear();
        counts.clear();
        for (int64_t i = 0; i < a[1]; ++i) {
          seqs.push_back(h[a[2 + 2 * i]]);
          counts.push_back(static_cast<int32_t>(a[3 + 2 * i]));
        }
        const int32_t n = static_cast<int32_t>(seqs.size());
        ++st.attend_calls;
        st.decode_queries += n;
        size_t need = 0;
        check(tkv_workspace_size(cache, seqs.data(), nullptr, n, &need), "tkv_workspace_size");
        if (host_) continue;
        if (need > ws_cap_) {
          if (ws_) hip_check(hipStreamSynchronize(stream_), "hipStreamSynchronize");
          if (ws_) (void)hipFree(ws_);
          ws_cap_ = need + need / 4;
          hip_check(hipMalloc(&ws_, ws_cap_), "hipMalloc");
        }
        // the tokens' K/V of this layer: the constant-filled source rows
        check(tkv_attend_decode_new_tokens(cache, static_cast<int32_t>(a[0]), seqs.data(), counts.data(), n, ksrc_,
                                           vsrc_, q_, static_cast<float*>(out_), ws_, ws_cap_, stream_),
              "tkv_attend_decode_new_tokens");
      } else if (op.kind == "verify_new") {
        // the reserved drafts' K/V of this layer (the constant-filled source
        // rows), written and verified in one call
        seqs.clear();
        counts.clear();
        int64_t rows = 0;
        for (int64_t i = 0; i < a[1]; ++i) {
          seqs.push_back(h[a[2 + 2 * i]]);
          counts.push_back(static_cast<int32_t>(a[3 + 2 * i]));
          rows += a[3 + 2 * i];
        }
        const int32_t n = static_cast<int32_t>(seqs.size());
        ++st.attend_calls;
        st.verify_tokens += rows;
        size_t need = 0;
        check(tkv_workspace_size(cache, seqs.data(), counts.data(), n, &need), "tkv_workspace_size");
        if (host_) continue;
        if (need > ws_cap_) {
          if (ws_) hip_check(hipStreamSynchronize(stream_), "hipStreamSynchronize");
          if (ws_) (void)hipFree(ws_);
          ws_cap_ = need + need / 4;
          hip_check(hipMalloc(&ws_, ws_cap_), "hipMalloc");
        }
        check(tkv_attend_verify_new_tokens(cache, static_cast<int32_t>(a[0]), seqs.data(), counts.data(), n, ksrc_,
                                           vsrc_, q_, static_cast<float*>(out_), ws_, ws_cap_, stream_),
              "tkv_attend_verify_new_tokens");
      } else if (op.kind == "fork") {
        const int32_t n = static_cast<int32_t>(a[1]);
        int64_t len = 0;
        check(tkv_seq_len(cache, h[a[0]], &len), "tkv_seq_len");
        seqs.resize(n);
        const auto f0 = std::chrono::steady_clock::now();
        check(tkv_fork(cache, h[a[0]], n, seqs.data()), "tkv_fork");
        st.fork_ns += std::chrono::duration<double, std::nano>(std::chrono::steady_clock::now() - f0).count();
        for (int32_t i = 0; i < n; ++i) h[a[2 + i]] = seqs[i];
        ++st.forks;
        st.full_copy_tokens += static_cast<int64_t>(n) * len;
      } else if (op.kind == "release") {
        check(tkv_release(cache, h[a[0]]), "tkv_release");
        h[a[0]] = 0;
      } else if (op.kind == "truncate") {
        check(tkv_truncate(cache, h[a[0]], a[1]), "tkv_truncate");
      } else if (op.kind == "decode" || op.kind == "verify") {
        const bool verify = op.kind == "verify";
        seqs.clear();
        counts.clear();
        int64_t rows = 0;
        for (int64_t i = 0; i < a[1]; ++i) {
          seqs.push_back(h[a[2 + (verify ? 2 * i : i)]]);
          if (verify) counts.push_back(static_cast<int32_t>(a[3 + 2 * i]));
          rows += verify ? a[3 + 2 * i] : 1;
        }
        const int32_t n = static_cast<int32_t>(seqs.size());
        const int32_t* nq = verify ? counts.data() : nullptr;
        ++st.attend_calls;
        (verify ? st.verify_tokens : st.decode_queries) += rows;
        size_t need = 0;
        check(tkv_workspace_size(cache, seqs.data(), nq, n, &need), "tkv_workspace_size");
        if (host_) continue;
        if (need > ws_cap_) {
          // only the first pass grows it, outside any timed region
          if (ws_) hip_check(hipStreamSynchronize(stream_), "hipStreamSynchronize");
          if (ws_) (void)hipFree(ws_);
          ws_cap_ = need + need / 4;
          hip_check(hipMalloc(&ws_, ws_cap_), "hipMalloc");
        }
        const int32_t layer = static_cast<int32_t>(a[0]);
        if (verify)
          check(tkv_attend_verify(cache, layer, seqs.data(), nq, n, q_, static_cast<float*>(out_), ws_, ws_cap_,
                                  stream_),
                "tkv_attend_verify");
        else
          check(tkv_attend_decode(cache, layer, seqs.data(), n, q_, static_cast<float*>(out_), ws_, ws_cap_,
                                  stream_),
                "tkv_attend_decode");
      } else {
        die("unknown operation", op.kind.c_str());
      }
    }
    sync();
    if (timed) {
      st.wall_ms = now_ms() - t0;
      if (measure && !host_) {
        int64_t calls = 0;
        check(tkv_profile_read(cache, &st.attend_ms, &st.merge_ms, &calls), "tkv_profile_read");
      }
      check(tkv_get_counters(cache, &st.counters), "tkv_get_counters");
      st.counters.plans_built -= base.plans_built;
      st.counters.plans_patched -= base.plans_patched;
      st.counters.plans_uploaded -= base.plans_uploaded;
      st.counters.plans_reused -= base.plans_reused;
    }
    // empty the cache for the next pass: release every live handle
    for (tkv_seq x : h)
      if (x) check(tkv_release(cache, x), "tkv_release");
    return st;
  }

  void sync() {
    if (!host_) hip_check(hipStreamSynchronize(stream_), "hipStreamSynchronize");
  }

  int64_t token_bytes() const { return static_cast<int64_t>(cfg_.layers) * cfg_.hkv * cfg_.d * elem_ * 2; }

 private:
  Config cfg_;
  const std::vector<Op>& ops_;
  bool host_ = false;
  size_t elem_ = 2, names_ = 1;
  hipStream_t stream_ = nullptr;
  void *kpool_ = nullptr, *vpool_ = nullptr, *ksrc_ = nullptr, *vsrc_ = nullptr, *q_ = nullptr, *out_ = nullptr;
  void* ws_ = nullptr;
  size_t ws_cap_ = 0;
  tkv_cache* cache_ = nullptr;
};

}  // namespace

int main(int argc, char** argv) {
  if (argc < 2) die("usage", "replay_bench OPS_FILE [--host]");
  const bool host = argc > 2 && std::string(argv[2]) == "--host";
  FILE* f = fopen(argv[1], "r");
  if (!f) die("cannot open", argv[1]);
  std::vector<Op> ops;
  Config cfg;
  char line[1 << 16];
  while (fgets(line, sizeof line, f)) {
    std::istringstream in(line);
    Op op;
    if (!(in >> op.kind)) continue;
    int64_t x;
    while (in >> x) op.a.push_back(x);
    if (op.kind == "config") {
      if (op.a.size() != 6) die("bad config line", line);
      cfg.layers = static_cast<int32_t>(op.a[0]);
      cfg.hq = static_cast<int32_t>(op.a[1]);
      cfg.hkv = static_cast<int32_t>(op.a[2]);
      cfg.d = static_cast<int32_t>(op.a[3]);
      cfg.blocks = static_cast<int32_t>(op.a[4]);
      cfg.bf16 = static_cast<int32_t>(op.a[5]);
      continue;
    }
    ops.push_back(op);
  }
  fclose(f);
  if (cfg.layers < 1) die("missing config line", argv[1]);
  Replayer r(cfg, ops, host);
  r.run(false);
  // wall time from a pass without the library's profiling events (they add
  // host work to every attention call); kernel times from one with them
  Stats s = r.run(false);
  const Stats prof = r.run(true);
  s.attend_ms = prof.attend_ms;
  s.merge_ms = prof.merge_ms;
  const int64_t tb = r.token_bytes();
  const int64_t block_bytes = 16 * tb;
  printf("{\"wall_ms\": %.4f, \"attend_calls\": %lld, \"decode_queries\": %lld, \"verify_tokens\": %lld, "
         "\"attend_kernel_ms\": %.4f, \"merge_kernel_ms\": %.4f, \"forks\": %lld, \"fork_ns\": %.1f, "
         "\"appended_tokens\": %lld, \"peak_blocks\": %lld, \"cow_peak_bytes\": %lld, \"full_copy_bytes\": %lld, "
         "\"plans_built\": %lld, \"plans_patched\": %lld, \"plans_uploaded\": %lld, \"plans_reused\": %lld}\n",
         s.wall_ms, static_cast<long long>(s.attend_calls), static_cast<long long>(s.decode_queries),
         static_cast<long long>(s.verify_tokens), s.attend_ms + s.merge_ms, s.merge_ms,
         static_cast<long long>(s.forks), s.forks ? s.fork_ns / s.forks : 0.0, static_cast<long long>(s.appended),
         static_cast<long long>(s.peak_blocks), static_cast<long long>(s.peak_blocks * block_bytes),
         static_cast<long long>(s.full_copy_tokens * tb), static_cast<long long>(s.counters.plans_built),
         static_cast<long long>(s.counters.plans_patched), static_cast<long long>(s.counters.plans_uploaded),
         static_cast<long long>(s.counters.plans_reused));
  return 0;
}
