// The C ABI: argument checks, plan caching and upload, kernel launches.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstddef>
#include <cstring>
#include <new>
#include <vector>

#include "kernels.h"
#include "plan.h"
#include "tkv.h"
#include "tree.h"

using namespace tkv;

namespace tkv {

namespace {
constexpr size_t kLaunchLogBytes = 1024;
thread_local char g_launch_log[kLaunchLogBytes];
thread_local size_t g_launch_log_len = 0;
}  // namespace

void launch_log_reset() {
  g_launch_log_len = 0;
  g_launch_log[0] = '\0';
}

void launch_log_add(const char* name) {
  const size_t n = std::strlen(name);
  const size_t sep = g_launch_log_len ? 1 : 0;
  if (g_launch_log_len + sep + n + 1 > kLaunchLogBytes) return;
  if (sep) g_launch_log[g_launch_log_len++] = ';';
  std::memcpy(g_launch_log + g_launch_log_len, name, n + 1);
  g_launch_log_len += n;
}

const char* launch_log() { return g_launch_log; }

}  // namespace tkv

namespace {

// A pinned host buffer a plan (or a list of changed words) is read from (p on
// the host, dp on the device); ev is recorded behind the launch or copy that
// reads it, busy until it has been waited for.
struct Staging {
  void* p = nullptr;
  void* dp = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool busy = false;
};

struct PlanSlot {
  std::vector<tkv_seq> seqs;
  std::vector<int32_t> nq;
  bool verify = false;
  uint64_t epoch = 0;
  uint64_t shape_epoch = 0;
  uint64_t opt_epoch = 0;
  bool valid = false;
  Plan plan;
  void* dev = nullptr;  // the serialised plan, then room for a list of changed words
  size_t dev_cap = 0;
  bool uploaded = false;  // dev holds the plan as of the last upload
  // words changed by patch_plan since that upload (uploaded == true only)
  std::vector<PlanWord> pending;
  // the device copy's words as the host last left them (small plans only;
  // empty = unknown): what a plan of the same shape for another batch is
  // compared with
  std::vector<uint32_t> shadow;
  // block ids the next attention launch on this plan writes into the device
  // copy (a reused device copy, see adopt_plan)
  std::vector<IdPatch> id_patches;
  uint64_t stamp = 0;
};

// Plans up to this size keep a host copy of their device words (PlanSlot::shadow).
constexpr size_t kShadowBytes = 64 << 10;

constexpr int kPlanSlots = 4;
// pinned staging buffers used in turn by plan uploads: a call waits only for
// the copy kStagings uploads back, so the host may run that far ahead of the GPU
constexpr int kStagings = 4;
// pinned staging made at tkv_create: the largest plan tkv_attend_decode_noalloc
// can upload without allocating (the 32-layer workload's decode plan is about
// 1.4 MiB)
constexpr size_t kStaticPlanStagingBytes = size_t(4) << 20;

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct DeviceGuard {
  int prev = -1;
  int want;
  explicit DeviceGuard(int dev) : want(dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != want) (void)hipSetDevice(want);
  }
  ~DeviceGuard() {
    if (prev >= 0 && prev != want) (void)hipSetDevice(prev);
  }
};

}  // namespace

struct tkv_cache {
  tkv_config cfg{};
  Tree tree;
  int device = -1;
  bool has_pools = false;
  PlanOptions opt;
  uint64_t opt_epoch = 1;
  bool plan_cache = true;
  bool plan_patch = true;  // TKV_OPT_PLAN_PATCH
  bool fuse_new = true;    // TKV_OPT_FUSED_NEW_TOKEN
  // a decode step's new tokens for the attention launch's arguments, and
  // tree node -> its tail entry in the call's plan (-1 between calls)
  NewTokens fused{};
  std::vector<int32_t> node_entry;
  int32_t waves = 0;
  int32_t cus = 256;  // compute units of the device (set at create when pools are given)
  int32_t concurrent = 0;  // TKV_OPT_CONCURRENT
  PlanSlot slots[kPlanSlots];
  PlanScratch scratch;
  Plan spare;                  // a plan is built here, then swapped into its slot
  std::vector<uint32_t> ser;   // the built plan's words, to compare with a shadow
  // tkv_append_batch's working lists, kept so a call of a familiar size
  // allocates nothing; seen[slot] == seen_stamp marks a handle of the batch
  std::vector<Placement> app_pl;
  std::vector<uint8_t> app_made;
  std::vector<AppendEntry> app_ents;
  std::vector<uint64_t> seen;
  uint64_t seen_stamp = 0;
  uint64_t stamp = 0;
  // pinned staging for plan uploads: a ring, and the noalloc path's own
  // buffer (made at tkv_create, never grown)
  Staging stg[kStagings];
  int stg_next = 0;
  Staging fixed_stg;
  // side streams (default priority) on which the kernel classes of one call
  // after the first run concurrently, forked from and joined back to the
  // caller's stream with events
  hipStream_t aux[kKernelClasses - 1] = {};
  hipEvent_t fork_ev = nullptr;
  hipEvent_t join_ev[kKernelClasses - 1] = {};
  // the kernels the last attention call launched (launch_log's format)
  char last_kernels[1024] = {0};
  // profiling
  bool prof = false;
  std::vector<std::array<hipEvent_t, 3>> prof_used;
  std::vector<hipEvent_t> ev_pool;
  int64_t prof_calls = 0;

  explicit tkv_cache(const tkv_config& c) : cfg(c), tree(c.num_blocks) {}

  size_t elem_bytes() const { return cfg.dtype == TKV_BF16 ? 2 : 4; }
  size_t tile_elems() const { return 16 * static_cast<size_t>(cfg.head_dim); }
  size_t layer_elems() const {
    return static_cast<size_t>(cfg.num_blocks) * cfg.num_kv_heads * tile_elems();
  }
  const char* kpool_layer(int layer) const {
    return static_cast<const char*>(cfg.k_pool) + layer * layer_elems() * elem_bytes();
  }
  const char* vpool_layer(int layer) const {
    return static_cast<const char*>(cfg.v_pool) + layer * layer_elems() * elem_bytes();
  }

  // Back to the pool, or destroyed when the pool cannot grow.
  void put_event(hipEvent_t e) {
    try {
      ev_pool.push_back(e);
    } catch (const std::bad_alloc&) {
      (void)hipEventDestroy(e);
    }
  }

  hipEvent_t get_event() {
    if (!ev_pool.empty()) {
      hipEvent_t e = ev_pool.back();
      ev_pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
};

namespace {

// Query positions (and their minima in the items) are read by the causal
// kernels only: a decode plan's device copy does not need them updated.
void drop_position_words(const Plan& p, std::vector<PlanWord>* words) {
  const size_t q0 = p.off_gqpos / 4, q1 = q0 + p.gqpos.size();
  const size_t i0 = p.off_items / 4, i1 = i0 + p.items.size() * (sizeof(DevItem) / 4);
  const size_t mp = offsetof(DevItem, min_pos) / 4;
  auto position = [&](const PlanWord& w) {
    return (w.word >= q0 && w.word < q1) || (w.word >= i0 && w.word < i1 && (w.word - i0) % (sizeof(DevItem) / 4) == mp);
  };
  words->erase(std::remove_if(words->begin(), words->end(), position), words->end());
}

void shadow_apply(PlanSlot* s, const PlanWord* w, size_t n) {
  if (s->shadow.empty()) return;
  for (size_t i = 0; i < n; ++i) {
    if (w[i].word >= s->shadow.size()) {
      s->shadow.clear();
      return;
    }
    s->shadow[w[i].word] = static_cast<uint32_t>(w[i].value);
  }
}

// A plan just built for a batch that no slot holds (c->spare) takes over the
// device copy of a cached plan of the same shape when the two differ only in
// block ids (the leaves under a search node at the depth of an earlier one):
// the slot then holds the new plan, and its next attention launch rewrites
// those ids in the device copy before reading them (id_patches) instead of
// the plan being uploaded.  Returns the slot, or nullptr.
PlanSlot* adopt_plan(tkv_cache* c) {
  const Plan& N = c->spare;
  if (!c->plan_patch || N.bytes > kShadowBytes || N.bytes % 4) return nullptr;
  const size_t nw = N.bytes / 4;
  try {
    c->ser.resize(nw);
  } catch (const std::bad_alloc&) {
    return nullptr;
  }
  std::memset(c->ser.data(), 0, N.bytes);
  N.serialise(c->ser.data());
  const uint32_t b0 = static_cast<uint32_t>(N.off_blocks / 4), per = sizeof(DevBlock) / 4;
  const uint32_t b1 = b0 + static_cast<uint32_t>(N.blocks.size()) * per;
  for (auto& s : c->slots) {
    const Plan& O = s.plan;
    if (!s.valid || !s.uploaded || !s.pending.empty() || !s.id_patches.empty() || s.shadow.size() != nw) continue;
    if (O.off_items != N.off_items || O.off_gq != N.off_gq || O.off_gqpos != N.off_gqpos ||
        O.off_blocks != N.off_blocks || O.off_parts != N.off_parts || O.off_merge != N.off_merge)
      continue;
    bool ok = true;
    s.id_patches.clear();
    for (size_t w = 0; w < nw && ok; ++w) {
      if (c->ser[w] == s.shadow[w]) continue;
      const uint32_t word = static_cast<uint32_t>(w);
      ok = word >= b0 && word < b1 && (word - b0) % per == 0 &&
           s.id_patches.size() < static_cast<size_t>(kMaxIdPatches);
      if (ok) s.id_patches.push_back(IdPatch{static_cast<int32_t>((word - b0) / per), static_cast<int32_t>(c->ser[w])});
    }
    if (!ok) {
      s.id_patches.clear();
      continue;
    }
    return &s;
  }
  return nullptr;
}

int find_plan(tkv_cache* c, const tkv_seq* seqs, const int32_t* nq, int32_t nseq, PlanSlot** out) {
  const bool verify = nq != nullptr;
  const uint64_t ep = c->tree.epoch(), shape = c->tree.shape_epoch();
  if (c->plan_cache) {
    for (auto& s : c->slots) {
      if (!s.valid || s.opt_epoch != c->opt_epoch || s.verify != verify) continue;
      // a plan made before appends that all fitted in their tip nodes' last
      // blocks is brought up to date in place instead of rebuilt
      const bool patch = s.epoch != ep && c->plan_patch && s.shape_epoch == shape;
      if (s.epoch != ep && !patch) continue;
      if (s.seqs.size() != static_cast<size_t>(nseq)) continue;
      if (std::memcmp(s.seqs.data(), seqs, nseq * sizeof(tkv_seq))) continue;
      if (verify && std::memcmp(s.nq.data(), nq, nseq * sizeof(int32_t))) continue;
      if (patch) {
        bool listed = false;
        if (s.uploaded && s.pending.empty()) {
          // the device copy is the plan as it stands: list the words that change
          try {
            patch_plan(c->tree, &s.plan, &s.pending);
            if (!s.plan.causal) drop_position_words(s.plan, &s.pending);
            listed = true;
          } catch (const std::bad_alloc&) {
            s.pending.clear();
          }
        }
        if (!listed) {
          // (patched again before an upload, or no memory for the list):
          // upload the whole plan
          patch_plan(c->tree, &s.plan, nullptr);
          s.pending.clear();
          s.uploaded = false;
        }
        s.epoch = ep;
        ++c->tree.counters.plans_patched;
      }
      s.stamp = ++c->stamp;
      *out = &s;
      return TKV_OK;
    }
  }
  // build (the spare plan, the planner's scratch and every slot's lists keep
  // their memory, so a build of a familiar size allocates nothing), then take
  // over a cached device copy of the same shape, or the least recently used
  // slot (a slot with stale contents first)
  const int32_t gsize = c->cfg.num_q_heads / c->cfg.num_kv_heads;
  if (int rc = build_plan(c->tree, seqs, nq, nseq, gsize, c->cfg.num_kv_heads, c->opt, &c->spare, &c->scratch))
    return rc;
  PlanSlot* victim = c->plan_cache ? adopt_plan(c) : nullptr;
  const bool adopted = victim != nullptr;
  if (!adopted) {
    victim = &c->slots[0];
    for (auto& s : c->slots) {
      const bool stale = !s.valid || s.epoch != ep || s.opt_epoch != c->opt_epoch;
      const bool vstale = !victim->valid || victim->epoch != ep || victim->opt_epoch != c->opt_epoch;
      if (stale && !vstale) victim = &s;
      else if (stale == vstale && s.stamp < victim->stamp) victim = &s;
    }
  }
  victim->valid = false;
  std::swap(victim->plan, c->spare);
  try {
    victim->seqs.assign(seqs, seqs + nseq);
    if (verify) victim->nq.assign(nq, nq + nseq);
    else victim->nq.clear();
  } catch (const std::bad_alloc&) {
    return TKV_E_NOMEM;
  }
  victim->verify = verify;
  victim->epoch = ep;
  victim->shape_epoch = shape;
  victim->pending.clear();
  victim->opt_epoch = c->opt_epoch;
  victim->valid = true;
  victim->stamp = ++c->stamp;
  ++c->tree.counters.plans_built;
  if (adopted) {
    // the device copy stays; its block ids change with the next launch
    ++c->tree.counters.plans_patched;
    ++c->tree.counters.plans_reused;
  } else {
    victim->uploaded = false;
    victim->id_patches.clear();
    victim->shadow.clear();
  }
  *out = victim;
  return TKV_OK;
}

// `g` holding at least `bytes`, once the copy that last read it is done.
int take_staging(Staging* g, size_t bytes) {
  if (g->busy) {
    if (hipEventSynchronize(g->ev) != hipSuccess) return TKV_E_DEVICE;
    g->busy = false;
  }
  if (g->cap < bytes) {
    if (g->p) (void)hipHostFree(g->p);
    g->p = g->dp = nullptr;
    g->cap = 0;
    const size_t cap = align256(bytes + bytes / 4);
    if (hipHostMalloc(&g->p, cap, hipHostMallocMapped) != hipSuccess) {
      g->p = nullptr;
      return TKV_E_NOMEM;
    }
    if (hipHostGetDevicePointer(&g->dp, g->p, 0) != hipSuccess) {
      (void)hipHostFree(g->p);
      g->p = g->dp = nullptr;
      return TKV_E_DEVICE;
    }
    g->cap = cap;
  }
  if (!g->ev && hipEventCreateWithFlags(&g->ev, hipEventDisableTiming) != hipSuccess) return TKV_E_DEVICE;
  return TKV_OK;
}

// The next staging buffer of the ring, holding at least `bytes`.
int stage(tkv_cache* c, size_t bytes, Staging** out) {
  Staging* g = &c->stg[c->stg_next];
  if (int rc = take_staging(g, bytes)) return rc;
  c->stg_next = (c->stg_next + 1) % kStagings;
  *out = g;
  return TKV_OK;
}

// Marks `g` as read by the copy just queued on `stream`.
int staged_copy_queued(Staging* g, hipStream_t stream) {
  if (hipEventRecord(g->ev, stream) != hipSuccess) return TKV_E_DEVICE;
  g->busy = true;
  return TKV_OK;
}

// The changed words of a patched plan: copied behind the plan in its device
// buffer, then written into it by a small kernel, in stream order after the
// kernels that read the plan before.
int upload_patch(tkv_cache* c, PlanSlot* s, hipStream_t stream) {
  const size_t n = s->pending.size();
  shadow_apply(s, s->pending.data(), n);
  const size_t bytes = n * sizeof(PlanWord);
  const uint32_t limit = static_cast<uint32_t>(s->plan.bytes / 4);
  for (const PlanWord& w : s->pending)
    if (w.word >= limit) return TKV_E_INVAL;
  char* dev = static_cast<char*>(s->dev);
  if (n <= 4 * static_cast<size_t>(kPatchArgWords)) {
    // a short list travels in the kernels' arguments: no copy to wait for
    for (size_t i0 = 0; i0 < n; i0 += kPatchArgWords) {
      PatchArgs a;
      a.plan = reinterpret_cast<int32_t*>(dev);
      a.n = static_cast<int32_t>(std::min<size_t>(kPatchArgWords, n - i0));
      a.limit = limit;
      std::memcpy(a.w, s->pending.data() + i0, a.n * sizeof(PlanWord));
      if (launch_plan_patch_args(a, stream) != hipSuccess) return TKV_E_DEVICE;
    }
    s->pending.clear();
    return TKV_OK;
  }
  // a longer one is read by the patch kernel from pinned staging
  Staging* g = nullptr;
  if (int rc = stage(c, bytes, &g)) return rc;
  std::memcpy(g->p, s->pending.data(), bytes);
  if (launch_plan_patch(reinterpret_cast<int32_t*>(dev), static_cast<const PlanWord*>(g->dp), static_cast<int32_t>(n),
                        limit, stream) != hipSuccess)
    return TKV_E_DEVICE;
  if (int rc = staged_copy_queued(g, stream)) return rc;
  s->pending.clear();
  return TKV_OK;
}

int upload_plan(tkv_cache* c, PlanSlot* s, hipStream_t stream) {
  if (s->uploaded && s->pending.empty()) return TKV_OK;
  const size_t bytes = align256(std::max<size_t>(s->plan.bytes, 256));
  if (s->uploaded && s->dev_cap >= bytes) return upload_patch(c, s, stream);
  s->pending.clear();
  s->uploaded = false;
  if (s->dev_cap < bytes) {
    if (s->dev) {
      // the old buffer may still be read by queued kernels
      if (hipStreamSynchronize(stream) != hipSuccess) return TKV_E_DEVICE;
      (void)hipFree(s->dev);
      s->dev = nullptr;
      s->dev_cap = 0;
    }
    const size_t cap = align256(bytes + bytes / 4);
    if (hipMalloc(&s->dev, cap) != hipSuccess) {
      s->dev = nullptr;
      return TKV_E_NOMEM;
    }
    s->dev_cap = cap;
  }
  Staging* g = nullptr;
  if (int rc = stage(c, std::max<size_t>(s->plan.bytes, 256), &g)) return rc;
  const bool keep = s->plan.bytes <= kShadowBytes && s->plan.bytes % 4 == 0;
  if (keep) std::memset(g->p, 0, s->plan.bytes);  // the gaps between sections too, as the shadow has them
  s->plan.serialise(g->p);
  s->id_patches.clear();
  s->shadow.clear();
  if (keep) {
    try {
      const uint32_t* w = static_cast<const uint32_t*>(g->p);
      s->shadow.assign(w, w + s->plan.bytes / 4);
    } catch (const std::bad_alloc&) {
      s->shadow.clear();
    }
  }
  // copied by a kernel in the caller's stream, which reads the staging over the
  // host link: the attention launch after it then starts without waiting for
  // a copy engine
  if (launch_plan_copy(s->dev, g->dp, s->plan.bytes, stream) != hipSuccess) return TKV_E_DEVICE;
  if (int rc = staged_copy_queued(g, stream)) return rc;
  s->uploaded = true;
  ++c->tree.counters.plans_uploaded;
  return TKV_OK;
}

size_t partial_bytes(const tkv_cache* c, const Plan& p) {
  if (p.partial_slots == 0) return 0;
  const size_t acc = align256(static_cast<size_t>(p.partial_slots) * c->cfg.head_dim * sizeof(float));
  return acc + align256(static_cast<size_t>(p.partial_slots) * 2 * sizeof(float));
}

// Before a decode call that writes its new tokens: the plan's device copy
// (a whole upload; or its changed words, carried by the preparation launch
// when they fit) and the tokens' K/V of this layer, in one launch per 128
// tokens.
int prepare_new_tokens(tkv_cache* c, PlanSlot* s, int32_t layer, int32_t nseq, const void* k_new,
                       const void* v_new, hipStream_t stream) {
  bool carry = false;
  if (!s->uploaded || s->pending.size() > static_cast<size_t>(kPrepPatchWords)) {
    if (int rc = upload_plan(c, s, stream)) return rc;
  } else {
    carry = !s->pending.empty();
  }
  const uint32_t limit = static_cast<uint32_t>(s->plan.bytes / 4);
  DecodePrepArgs a{};
  a.app.src_k = k_new;
  a.app.src_v = v_new;
  a.app.kpool = const_cast<char*>(c->kpool_layer(layer));
  a.app.vpool = const_cast<char*>(c->vpool_layer(layer));
  a.app.layer_stride = 0;
  a.app.ntok = 0;
  for (int32_t i = 0; i < nseq; ++i) a.app.ntok += c->app_ents[i].cnt;
  a.app.hkv = c->cfg.num_kv_heads;
  a.plan = static_cast<int32_t*>(s->dev);
  a.limit = limit;
  const std::vector<AppendEntry>& ents = c->app_ents;
  for (int32_t e0 = 0; e0 < nseq; e0 += kAppendMaxBlocks) {
    a.app.nent = std::min(kAppendMaxBlocks, nseq - e0);
    for (int32_t i = 0; i < a.app.nent; ++i) a.app.ent[i] = ents[e0 + i];
    a.npatch = 0;
    if (e0 == 0 && carry) {
      for (const PlanWord& w : s->pending)
        if (w.word >= limit) return TKV_E_INVAL;
      a.npatch = static_cast<int32_t>(s->pending.size());
      std::memcpy(a.patch, s->pending.data(), s->pending.size() * sizeof(PlanWord));
      shadow_apply(s, s->pending.data(), s->pending.size());
    }
    if (launch_decode_prep(c->cfg.dtype, c->cfg.head_dim, a, stream) != hipSuccess) return TKV_E_DEVICE;
  }
  if (carry) s->pending.clear();
  return TKV_OK;
}

// A decode step whose new tokens the attention launch writes itself: possible
// when the plan lists at most kFusedMaxTokens tail blocks (one token record
// each), every handle's new tokens lie in its tip block as listed by the
// plan, and the plan's device copy is either uploaded whole first or differs
// from the host plan only in those blocks' valid counts (which the launch
// writes too).  Fills c->fused and uploads the plan
// if needed; returns false (nothing done) when the preparation launch must
// write them instead.
bool prepare_fused(tkv_cache* c, PlanSlot* s, int32_t layer, const tkv_seq* seqs, int32_t nseq, const void* k_new,
                   const void* v_new, int* rc) {
  *rc = TKV_OK;
  const Plan& P = s->plan;
  // the launch's token list is indexed by the plan's tail blocks (DevItem::tails)
  const int32_t ntail = static_cast<int32_t>(P.tail_entry.size());
  if (!c->fuse_new || ntail > kFusedMaxTokens) return false;
  // a workgroup holds its item's token records in one wave's lanes
  for (const DevItem& it : P.items)
    if ((it.tails >> 16) > 64) return false;
  try {
    if (c->node_entry.size() < static_cast<size_t>(c->tree.node_capacity()))
      c->node_entry.resize(c->tree.node_capacity(), -1);
  } catch (const std::bad_alloc&) {
    return false;
  }
  NewTokens& x = c->fused;
  for (int32_t t = 0; t < ntail; ++t) {
    c->node_entry[P.tail_node[t]] = t;
    x.tok[t] = NewTok{-1, 0, 0, 0, 0};
  }
  bool ok = true;
  for (int32_t i = 0; i < nseq && ok; ++i) {
    int32_t tip = -1;
    const AppendEntry& a = c->app_ents[i];
    if (c->tree.resolve(seqs[i], &tip) != TKV_OK) {
      ok = false;
      break;
    }
    const int32_t t = c->node_entry[tip];
    const int32_t e = t >= 0 ? P.tail_entry[t] : -1;
    if (e < 0 || P.blocks[e].id != a.blk || P.blocks[e].valid != a.slot + a.cnt || x.tok[t].entry >= 0) {
      ok = false;
      break;
    }
    x.tok[t] = NewTok{e, a.blk, static_cast<int16_t>(a.slot), static_cast<int16_t>(a.cnt), a.src};
  }
  for (int32_t t = 0; t < ntail; ++t) c->node_entry[P.tail_node[t]] = -1;
  if (!ok) return false;
  if (s->uploaded && !s->pending.empty()) {
    // every changed word must be one the launch writes: a new token's valid count
    const uint32_t v0 = static_cast<uint32_t>((P.off_blocks + offsetof(DevBlock, valid)) / 4);
    const uint32_t per = sizeof(DevBlock) / 4;
    for (const PlanWord& w : s->pending) {
      bool covered = false;
      if (w.word >= v0 && (w.word - v0) % per == 0) {
        const int32_t e = static_cast<int32_t>((w.word - v0) / per);
        for (int32_t t = 0; t < ntail && !covered; ++t)
          covered = x.tok[t].entry == e && w.value == x.tok[t].slot + x.tok[t].n;
      }
      if (!covered) return false;
    }
  }
  x.multi = 0;
  for (int32_t t = 0; t < ntail; ++t) x.multi |= x.tok[t].n > 1 ? 1 : 0;
  x.k = k_new;
  x.v = v_new;
  x.kpool = const_cast<char*>(c->kpool_layer(layer));
  x.vpool = const_cast<char*>(c->vpool_layer(layer));
  x.n = ntail;
  return true;
}

// The plan of a tkv_attend_decode_noalloc call, copied into the fixed device
// workspace `base` from the pinned staging made for it at tkv_create (no
// allocation: a plan larger than that staging is refused).
int upload_plan_fixed(tkv_cache* c, const Plan& P, char* base, hipStream_t stream) {
  Staging* g = &c->fixed_stg;
  if (P.bytes > g->cap || !g->ev) return TKV_E_WORKSPACE;
  if (int rc = take_staging(g, P.bytes)) return rc;
  P.serialise(g->p);
  if (hipMemcpyAsync(base, g->p, P.bytes, hipMemcpyHostToDevice, stream) != hipSuccess) return TKV_E_DEVICE;
  return staged_copy_queued(g, stream);
}

// fixed_ws: the call's plan and partial records go to the device's fixed
// workspace (tkv_attend_decode_noalloc) instead of the cached plan's buffer
// and the caller's workspace; nothing is allocated and no events are kept.
int attend(tkv_cache* c, int32_t layer, const tkv_seq* seqs, const int32_t* nq, int32_t nseq,
           const void* q, float* out, void* ws, size_t ws_bytes, void* stream_,
           const void* k_new = nullptr, const void* v_new = nullptr, bool fixed_ws = false,
           const int32_t* ntok = nullptr) {
  if (!c) return TKV_E_INVAL;
  if (!c->has_pools) return TKV_E_NODEVICE;
  if (layer < 0 || layer >= c->cfg.num_layers) return TKV_E_RANGE;
  if (!seqs || nseq < 1 || !q || !out) return TKV_E_INVAL;
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(ws) |
       reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new)) & 15)
    return TKV_E_INVAL;
  if ((k_new == nullptr) != (v_new == nullptr)) return TKV_E_INVAL;
  if (k_new) {
    // every handle once (two writes to one slot would race), and where its
    // last token lives
    try {
      if (c->seen.size() < c->tree.handle_slots()) c->seen.resize(c->tree.handle_slots() * 2, 0);
      c->app_ents.resize(nseq);
    } catch (const std::bad_alloc&) {
      return TKV_E_NOMEM;
    }
    const uint64_t stamp = ++c->seen_stamp;
    int32_t row = 0;
    for (int32_t i = 0; i < nseq; ++i) {
      // the handle's last n tokens: all in its last block, in its own tip node
      const int32_t n = ntok ? ntok[i] : 1;
      if (n < 1 || n > 16) return TKV_E_RANGE;
      int32_t blk, slot;
      if (int rc = c->tree.own_last_token(seqs[i], &blk, &slot)) return rc;
      if (slot - n + 1 < 0) return TKV_E_RANGE;
      uint64_t& mark = c->seen[Tree::slot_of(seqs[i])];
      if (mark == stamp) return TKV_E_INVAL;
      mark = stamp;
      c->app_ents[i] = {blk, slot - n + 1, row, n};
      row += n;
    }
  }
  PlanSlot* s = nullptr;
  if (int rc = find_plan(c, seqs, nq, nseq, &s)) return rc;
  const Plan& P = s->plan;
  const size_t need = partial_bytes(c, P);
  char* fixed = nullptr;
  if (fixed_ws) {
    fixed = static_cast<char*>(static_workspace(c->device));
    if (!fixed) return TKV_E_DEVICE;
    if (align256(P.bytes) + need > kStaticWorkspaceBytes) return TKV_E_WORKSPACE;
    ws = fixed + align256(P.bytes);
  } else if (need > 0 && (!ws || ws_bytes < need)) {
    return TKV_E_WORKSPACE;
  }
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  DeviceGuard dg(c->device);
  launch_log_reset();
  NewTokens* nt = nullptr;
  // block ids of a reused device copy (adopt_plan): written by the attention
  // launch when every kernel of the call is the register kernel, else by the
  // patch kernel with the other changed words
  const uint32_t b0 = static_cast<uint32_t>(P.off_blocks / 4), per = sizeof(DevBlock) / 4;
  bool ids_in_launch = false;
  if (!fixed && !s->id_patches.empty()) {
    ids_in_launch = true;
    for (int cls = 0; cls < kKernelClasses; ++cls) {
      if (P.bucket_begin[cls + 1] == P.bucket_begin[cls]) continue;
      const int64_t wgs = static_cast<int64_t>(P.bucket_begin[cls + 1] - P.bucket_begin[cls]) * c->cfg.num_kv_heads;
      if (cls >= 2 || (cls == 0 && !c->waves && wgs > c->cus)) ids_in_launch = false;
    }
    if (!ids_in_launch) {
      try {
        for (const IdPatch& ip : s->id_patches)
          s->pending.push_back(PlanWord{b0 + static_cast<uint32_t>(ip.entry) * per, ip.id});
      } catch (const std::bad_alloc&) {
        s->uploaded = false;  // uploaded whole instead
        s->pending.clear();
      }
      s->id_patches.clear();
    }
  }
  if (fixed) {
    if (int rc = upload_plan_fixed(c, P, fixed, stream)) return rc;
  } else if (k_new) {
    int rc = TKV_OK;
    if (prepare_fused(c, s, layer, seqs, nseq, k_new, v_new, &rc)) {
      // the plan's device copy: whole if it was never uploaded; otherwise it
      // differs only in the valid counts (and block ids) the launch writes
      if (!s->uploaded) {
        if (int rc2 = upload_plan(c, s, stream)) return rc2;
      }
      shadow_apply(s, s->pending.data(), s->pending.size());
      s->pending.clear();
      nt = &c->fused;
      nt->nid = 0;
    } else {
      if (ids_in_launch) {
        // the preparation launch carries the ids with the other changed words
        try {
          for (const IdPatch& ip : s->id_patches)
            s->pending.push_back(PlanWord{b0 + static_cast<uint32_t>(ip.entry) * per, ip.id});
        } catch (const std::bad_alloc&) {
          s->uploaded = false;
          s->pending.clear();
        }
        s->id_patches.clear();
        ids_in_launch = false;
      }
      if (int rc2 = prepare_new_tokens(c, s, layer, nseq, k_new, v_new, stream)) return rc2;
    }
  } else if (int rc = upload_plan(c, s, stream)) {
    return rc;
  }
  if (ids_in_launch && !s->id_patches.empty()) {
    if (!nt) {
      nt = &c->fused;
      nt->n = 0;
      nt->multi = 0;
    }
    nt->nid = static_cast<int32_t>(s->id_patches.size());
    std::memcpy(nt->ids, s->id_patches.data(), s->id_patches.size() * sizeof(IdPatch));
    for (const IdPatch& ip : s->id_patches)
      if (!s->shadow.empty()) s->shadow[b0 + static_cast<uint32_t>(ip.entry) * per] = static_cast<uint32_t>(ip.id);
    s->id_patches.clear();
  } else if (nt) {
    nt->nid = 0;
  }

  const char* dev = fixed ? fixed : static_cast<const char*>(s->dev);
  if (nt) nt->blocks = reinterpret_cast<DevBlock*>(const_cast<char*>(dev) + P.off_blocks);
  AttnArgs a{};
  a.kpool = c->kpool_layer(layer);
  a.vpool = c->vpool_layer(layer);
  a.q = q;
  a.out = out;
  a.items = reinterpret_cast<const DevItem*>(dev + P.off_items);
  a.gq = reinterpret_cast<const int32_t*>(dev + P.off_gq);
  a.gqpos = reinterpret_cast<const int32_t*>(dev + P.off_gqpos);
  a.blocks = reinterpret_cast<const DevBlock*>(dev + P.off_blocks);
  a.part_acc = static_cast<float*>(ws);
  a.part_ml = P.partial_slots
                  ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                             align256(static_cast<size_t>(P.partial_slots) * c->cfg.head_dim * 4))
                  : nullptr;
  a.hq = c->cfg.num_q_heads;
  a.hkv = c->cfg.num_kv_heads;
  a.gsize = a.hq / a.hkv;
  a.scale_log2 = static_cast<float>(1.4426950408889634 / std::sqrt(static_cast<double>(c->cfg.head_dim)));

  std::array<hipEvent_t, 3> ev{nullptr, nullptr, nullptr};
  const bool prof = c->prof && !fixed;
  if (prof) {
    for (auto& e : ev) e = c->get_event();
    if (ev[0] && ev[1] && ev[2]) (void)hipEventRecord(ev[0], stream);
  }
  // The kernel classes of this call, run by c->concurrent: 0 = one after
  // another on the caller's stream; 1 = the first on the caller's stream, each
  // further one on a side stream forked from it with an event and joined back
  // before the merge.
  int classes[kKernelClasses];
  int ncls = 0;
  for (int cls = 0; cls < kKernelClasses; ++cls)
    if (P.bucket_begin[cls + 1] > P.bucket_begin[cls]) classes[ncls++] = cls;
  const bool side = c->concurrent == 1 && ncls > 1 && !fixed;
  if (side) {
    if (!c->fork_ev && hipEventCreateWithFlags(&c->fork_ev, hipEventDisableTiming) != hipSuccess) return TKV_E_DEVICE;
    for (int k = 0; k < ncls - 1; ++k) {
      if (!c->aux[k] && hipStreamCreateWithFlags(&c->aux[k], hipStreamNonBlocking) != hipSuccess) return TKV_E_DEVICE;
      if (!c->join_ev[k] && hipEventCreateWithFlags(&c->join_ev[k], hipEventDisableTiming) != hipSuccess)
        return TKV_E_DEVICE;
    }
    if (hipEventRecord(c->fork_ev, stream) != hipSuccess) return TKV_E_DEVICE;
  }
  for (int k = 0; k < ncls; ++k) {
    const int cls = classes[k];
    const int32_t n = P.bucket_begin[cls + 1] - P.bucket_begin[cls];
    hipStream_t st = side && k > 0 ? c->aux[k - 1] : stream;
    if (st != stream && hipStreamWaitEvent(st, c->fork_ev, 0) != hipSuccess) return TKV_E_DEVICE;
    a.item0 = P.bucket_begin[cls];
    a.max_blocks = P.bucket_max_blocks[cls];
    hipError_t e;
    const int64_t wgs = static_cast<int64_t>(n) * c->cfg.num_kv_heads;
    if (cls == 0 && !c->waves && wgs > c->cus) {
      // One tile, more workgroups than CUs (a search tree's private nodes, a
      // large batch of sequences): the LDS-staged kernel's 4-tile shape,
      // whose shallow ring with two workgroups per CU streams these faster
      // than the register kernel
      e = launch_attn_rows(c->cfg.dtype, c->cfg.head_dim, 1, P.causal, a, n, st, c->cus, nt);
    } else if (cls < 2) {
      // One tile otherwise: two waves, i.e. few long streams of loads per CU,
      // which HBM serves faster than more, shorter ones; two tiles: four.
      const int w = c->waves ? c->waves : (cls == 0 ? 2 : 4);
      e = launch_attn_partial(c->cfg.dtype, c->cfg.head_dim, P.bucket_tiles[cls], w, P.causal, a, n, st, nt);
    } else {
      e = launch_attn_rows(c->cfg.dtype, c->cfg.head_dim, P.bucket_tiles[cls], P.causal, a, n, st, c->cus, nt);
    }
    if (e != hipSuccess) return TKV_E_DEVICE;
    if (st != stream && hipEventRecord(c->join_ev[k - 1], st) != hipSuccess) return TKV_E_DEVICE;
  }
  if (side)
    for (int k = 1; k < ncls; ++k)
      if (hipStreamWaitEvent(stream, c->join_ev[k - 1], 0) != hipSuccess) return TKV_E_DEVICE;
  if (prof && ev[1]) (void)hipEventRecord(ev[1], stream);
  if (P.any_merge) {
    MergeArgs m{};
    m.parts = reinterpret_cast<const DevPart*>(dev + P.off_parts);
    m.merge = reinterpret_cast<const DevMerge*>(dev + P.off_merge);
    m.part_acc = a.part_acc;
    m.part_ml = a.part_ml;
    m.out = out;
    m.hq = a.hq;
    m.nq = P.nqueries;
    m.scale_log2 = a.scale_log2;
    if (launch_attn_merge(c->cfg.head_dim, m, stream) != hipSuccess) return TKV_E_DEVICE;
  }
  std::memcpy(c->last_kernels, launch_log(), std::strlen(launch_log()) + 1);
  if (prof) {
    bool kept = false;
    if (ev[0] && ev[1] && ev[2]) {
      (void)hipEventRecord(ev[2], stream);
      try {
        c->prof_used.push_back(ev);
        ++c->prof_calls;
        kept = true;
      } catch (const std::bad_alloc&) {
        // no room to keep this call's events: it goes untimed
      }
    }
    if (!kept)
      for (auto e : ev)
        if (e) c->put_event(e);
  }
  return TKV_OK;
}

}  // namespace

extern "C" {

const char* tkv_strerror(int status) {
  switch (status) {
    case TKV_OK: return "ok";
    case TKV_E_INVAL: return "invalid argument";
    case TKV_E_NOMEM: return "out of blocks or memory";
    case TKV_E_BADSEQ: return "stale or unknown sequence handle";
    case TKV_E_SHARED: return "truncation would remove tokens shared with other branches";
    case TKV_E_EMPTY: return "attention over an empty sequence";
    case TKV_E_RANGE: return "value out of range";
    case TKV_E_DEVICE: return "HIP call or kernel launch failed";
    case TKV_E_WORKSPACE: return "workspace too small";
    case TKV_E_NODEVICE: return "cache has no device pools";
    default: return "unknown status";
  }
}

int tkv_create(const tkv_config* cfg, tkv_cache** out) {
  if (!cfg || !out) return TKV_E_INVAL;
  const tkv_config& c = *cfg;
  if (c.num_layers < 1 || c.num_q_heads < 1 || c.num_kv_heads < 1 || c.num_blocks < 1 ||
      c.num_blocks > kMaxPoolBlocks)
    return TKV_E_INVAL;
  if (c.num_q_heads % c.num_kv_heads || c.num_q_heads / c.num_kv_heads > kMaxRows) return TKV_E_INVAL;
  if (c.head_dim != 64 && c.head_dim != 128) return TKV_E_INVAL;
  if (c.block_size != kBlock || c.reserved != 0) return TKV_E_INVAL;
  if (c.dtype != TKV_F32 && c.dtype != TKV_BF16) return TKV_E_INVAL;
  if ((c.k_pool == nullptr) != (c.v_pool == nullptr)) return TKV_E_INVAL;
  if ((reinterpret_cast<uintptr_t>(c.k_pool) | reinterpret_cast<uintptr_t>(c.v_pool)) & 15) return TKV_E_INVAL;
  tkv_cache* cache = nullptr;
  try {
    cache = new tkv_cache(c);
  } catch (const std::bad_alloc&) {
    return TKV_E_NOMEM;
  }
  cache->has_pools = c.k_pool != nullptr;
  // the LDS-staged shapes' workgroups per CU (attn_rows.hip): fp32 at d = 128
  // takes a CU's registers with one
  cache->opt.two_per_cu = (c.dtype == TKV_BF16 || c.head_dim <= 64) ? 1 : 0;
  if (cache->has_pools) {
    int cus = 0;
    if (hipGetDevice(&cache->device) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, cache->device) != hipSuccess) {
      delete cache;
      return TKV_E_DEVICE;
    }
    if (cus > 0) cache->opt.target_wgs = cache->cus = cus;
    // set-up for tkv_attend_decode_noalloc: this device's fixed workspace and
    // the cache's pinned staging for its plans
    if (static_workspace_init(cache->device) || take_staging(&cache->fixed_stg, kStaticPlanStagingBytes)) {
      tkv_destroy(cache);
      return TKV_E_DEVICE;
    }
  }
  *out = cache;
  return TKV_OK;
}

int tkv_destroy(tkv_cache* c) {
  if (!c) return TKV_E_INVAL;
  if (c->has_pools) {
    DeviceGuard dg(c->device);
    (void)hipDeviceSynchronize();
    for (auto& s : c->slots)
      if (s.dev) (void)hipFree(s.dev);
    auto free_staging = [](Staging& g) {
      if (g.p) (void)hipHostFree(g.p);
      if (g.ev) (void)hipEventDestroy(g.ev);
    };
    for (Staging& g : c->stg) free_staging(g);
    free_staging(c->fixed_stg);
    for (auto& t : c->prof_used)
      for (auto e : t) (void)hipEventDestroy(e);
    for (auto e : c->ev_pool) (void)hipEventDestroy(e);
    for (auto& st : c->aux)
      if (st) (void)hipStreamDestroy(st);
    for (auto& e : c->join_ev)
      if (e) (void)hipEventDestroy(e);
    if (c->fork_ev) (void)hipEventDestroy(c->fork_ev);
  }
  delete c;
  return TKV_OK;
}

int tkv_seq_new(tkv_cache* c, tkv_seq* out) { return c ? c->tree.seq_new(out) : TKV_E_INVAL; }

int tkv_fork(tkv_cache* c, tkv_seq parent, int32_t n, tkv_seq* out_children) {
  return c ? c->tree.fork(parent, n, out_children) : TKV_E_INVAL;
}

int tkv_release(tkv_cache* c, tkv_seq s) { return c ? c->tree.release(s) : TKV_E_INVAL; }

int tkv_truncate(tkv_cache* c, tkv_seq s, int64_t new_len) {
  return c ? c->tree.truncate(s, new_len) : TKV_E_INVAL;
}

int tkv_append(tkv_cache* c, tkv_seq s, int32_t ntok, const void* k, const void* v, void* stream_) {
  return tkv_append_batch(c, &s, &ntok, 1, k, v, stream_);
}

int tkv_append_batch(tkv_cache* c, const tkv_seq* seqs, const int32_t* ntok, int32_t nseq, const void* k,
                     const void* v, void* stream_) {
  if (!c || !seqs || !ntok || nseq < 1) return TKV_E_INVAL;
  if ((k == nullptr) != (v == nullptr)) return TKV_E_INVAL;
  if (k && !c->has_pools) return TKV_E_NODEVICE;
  if (k && ((reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15)) return TKV_E_INVAL;
  std::vector<Placement>& pls = c->app_pl;
  std::vector<uint8_t>& made = c->app_made;
  std::vector<AppendEntry>& ents = c->app_ents;
  try {
    // everything that could refuse the batch is checked before any change:
    // handles, counts, repeats (two appends to one handle would write one
    // block from two workgroups), the source size and the free blocks
    if (c->seen.size() < c->tree.handle_slots()) c->seen.resize(c->tree.handle_slots() * 2, 0);
    const uint64_t stamp = ++c->seen_stamp;
    int64_t need = 0, total = 0;
    for (int32_t i = 0; i < nseq; ++i) {
      int64_t b = 0;
      if (int rc = c->tree.append_need(seqs[i], ntok[i], &b)) return rc;
      uint64_t& mark = c->seen[Tree::slot_of(seqs[i])];
      if (mark == stamp) return TKV_E_INVAL;
      mark = stamp;
      need += b;
      total += ntok[i];
    }
    if (total > INT32_MAX) return TKV_E_RANGE;
    if (need > c->tree.num_free()) return TKV_E_NOMEM;
    if (pls.size() < static_cast<size_t>(nseq)) pls.resize(nseq);
    made.resize(nseq);
    ents.clear();
    ents.reserve(static_cast<size_t>(need + nseq));
  } catch (const std::bad_alloc&) {
    return TKV_E_NOMEM;
  }
  auto undo = [&](int32_t upto) {
    for (int32_t i = upto - 1; i >= 0; --i) c->tree.undo_append(seqs[i], ntok[i], pls[i], made[i] != 0);
  };
  int32_t src = 0;
  for (int32_t i = 0; i < nseq; ++i) {
    if (int rc = c->tree.append(seqs[i], ntok[i], &pls[i])) {
      undo(i);
      return rc;
    }
    made[i] = c->tree.last_append_made_node() ? 1 : 0;
    // the blocks it writes: the first from its first free slot, the rest whole
    const Placement& pl = pls[i];
    int32_t done = 0;
    for (size_t j = 0; j < pl.blocks.size(); ++j) {
      const int32_t slot = j == 0 ? pl.first_slot : 0;
      const int32_t cnt = std::min(16 - slot, ntok[i] - done);
      ents.push_back({pl.blocks[j], slot, src + done, cnt});
      done += cnt;
    }
    src += ntok[i];
  }
  if (!k) return TKV_OK;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  DeviceGuard dg(c->device);
  const int32_t nent = static_cast<int32_t>(ents.size());
  for (int32_t e0 = 0; e0 < nent; e0 += kAppendWideBlocks) {
    AppendArgs a{};
    a.src_k = k;
    a.src_v = v;
    a.kpool = c->cfg.k_pool;
    a.vpool = c->cfg.v_pool;
    a.layer_stride = static_cast<int64_t>(c->layer_elems());
    a.ntok = src;
    a.hkv = c->cfg.num_kv_heads;
    a.nent = std::min(kAppendWideBlocks, nent - e0);
    for (int32_t i = 0; i < a.nent; ++i) a.ent[i] = ents[e0 + i];
    if (launch_append(c->cfg.dtype, c->cfg.head_dim, c->cfg.num_layers, a, stream) != hipSuccess) {
      undo(nseq);
      return TKV_E_DEVICE;
    }
  }
  return TKV_OK;
}

int tkv_workspace_size(tkv_cache* c, const tkv_seq* seqs, const int32_t* nq, int32_t nseq, size_t* bytes) {
  if (!c || !bytes) return TKV_E_INVAL;
  PlanSlot* s = nullptr;
  if (int rc = find_plan(c, seqs, nq, nseq, &s)) return rc;
  *bytes = partial_bytes(c, s->plan);
  return TKV_OK;
}

int tkv_attend_decode(tkv_cache* c, int32_t layer, const tkv_seq* seqs, int32_t nseq, const void* q,
                      float* out, void* ws, size_t ws_bytes, void* stream) {
  return attend(c, layer, seqs, nullptr, nseq, q, out, ws, ws_bytes, stream);
}

int tkv_attend_decode_new_token(tkv_cache* c, int32_t layer, const tkv_seq* seqs, int32_t nseq, const void* k_new,
                                const void* v_new, const void* q, float* out, void* ws, size_t ws_bytes,
                                void* stream) {
  if (!k_new || !v_new) return TKV_E_INVAL;
  return attend(c, layer, seqs, nullptr, nseq, q, out, ws, ws_bytes, stream, k_new, v_new);
}

int tkv_attend_decode_new_tokens(tkv_cache* c, int32_t layer, const tkv_seq* seqs, const int32_t* ntok,
                                 int32_t nseq, const void* k_new, const void* v_new, const void* q, float* out,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (!k_new || !v_new || !ntok) return TKV_E_INVAL;
  return attend(c, layer, seqs, nullptr, nseq, q, out, ws, ws_bytes, stream, k_new, v_new, false, ntok);
}

int tkv_attend_verify_new_tokens(tkv_cache* c, int32_t layer, const tkv_seq* seqs, const int32_t* nq, int32_t nseq,
                                 const void* k_new, const void* v_new, const void* q, float* out, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!k_new || !v_new || !nq) return TKV_E_INVAL;
  // the verified tokens are the new ones: handle i's last nq[i]
  return attend(c, layer, seqs, nq, nseq, q, out, ws, ws_bytes, stream, k_new, v_new, false, nq);
}

int tkv_attend_decode_noalloc(tkv_cache* c, int32_t layer, const tkv_seq* seqs, int32_t nseq, const void* q,
                              float* out, void* stream) {
  return attend(c, layer, seqs, nullptr, nseq, q, out, nullptr, 0, stream, nullptr, nullptr, true);
}

int tkv_attend_verify(tkv_cache* c, int32_t layer, const tkv_seq* seqs, const int32_t* nq, int32_t nseq,
                      const void* q, float* out, void* ws, size_t ws_bytes, void* stream) {
  if (!nq) return TKV_E_INVAL;
  return attend(c, layer, seqs, nq, nseq, q, out, ws, ws_bytes, stream);
}

int tkv_gather(tkv_cache* c, tkv_seq s, int32_t layer, void* k_out, void* v_out, void* stream_) {
  if (!c) return TKV_E_INVAL;
  if (!c->has_pools) return TKV_E_NODEVICE;
  if (layer < 0 || layer >= c->cfg.num_layers) return TKV_E_RANGE;
  if (!k_out || !v_out) return TKV_E_INVAL;
  if ((reinterpret_cast<uintptr_t>(k_out) | reinterpret_cast<uintptr_t>(v_out)) & 15) return TKV_E_INVAL;
  int32_t n = 0;
  int rc = c->tree.block_table(s, nullptr, nullptr, 0, &n);
  if (rc && rc != TKV_E_RANGE) return rc;
  std::vector<int32_t> ids, valid;
  try {
    ids.resize(n);
    valid.resize(n);
  } catch (const std::bad_alloc&) {
    return TKV_E_NOMEM;
  }
  if (n > 0 && (rc = c->tree.block_table(s, ids.data(), valid.data(), n, &n))) return rc;
  hipStream_t stream = static_cast<hipStream_t>(stream_);
  DeviceGuard dg(c->device);
  int32_t pos = 0;
  for (int32_t e0 = 0; e0 < n; e0 += kGatherMaxBlocks) {
    GatherArgs a{};
    a.kpool = c->kpool_layer(layer);
    a.vpool = c->vpool_layer(layer);
    a.k_out = k_out;
    a.v_out = v_out;
    a.hkv = c->cfg.num_kv_heads;
    a.nent = std::min(kGatherMaxBlocks, n - e0);
    for (int32_t i = 0; i < a.nent; ++i) {
      a.blk[i] = ids[e0 + i];
      a.valid[i] = valid[e0 + i];
      a.pos[i] = pos;
      pos += valid[e0 + i];
    }
    if (launch_gather(c->cfg.dtype, c->cfg.head_dim, a, stream) != hipSuccess) return TKV_E_DEVICE;
  }
  return TKV_OK;
}

int tkv_seq_len(const tkv_cache* c, tkv_seq s, int64_t* len) { return c ? c->tree.seq_len(s, len) : TKV_E_INVAL; }

int tkv_block_table(const tkv_cache* c, tkv_seq s, int32_t* ids, int32_t* valid, int32_t cap, int32_t* n) {
  return c ? c->tree.block_table(s, ids, valid, cap, n) : TKV_E_INVAL;
}

int tkv_block_refcount(const tkv_cache* c, int32_t block, int32_t* rc) {
  return c ? c->tree.block_refcount(block, rc) : TKV_E_INVAL;
}

int tkv_block_refcounts(const tkv_cache* c, int32_t* rc) { return c ? c->tree.block_refcounts(rc) : TKV_E_INVAL; }

int tkv_num_free(const tkv_cache* c, int32_t* n) {
  if (!c || !n) return TKV_E_INVAL;
  *n = c->tree.num_free();
  return TKV_OK;
}

int tkv_last_kernels(const tkv_cache* c, char* buf, int32_t cap) {
  if (!c || !buf || cap < 1) return TKV_E_INVAL;
  const size_t n = std::strlen(c->last_kernels);
  const size_t k = std::min(n, static_cast<size_t>(cap) - 1);
  std::memcpy(buf, c->last_kernels, k);
  buf[k] = '\0';
  return k == n ? TKV_OK : TKV_E_RANGE;
}

int tkv_get_counters(const tkv_cache* c, tkv_counters* out) {
  if (!c || !out) return TKV_E_INVAL;
  *out = c->tree.counters;
  return TKV_OK;
}

int tkv_plan_info_get(tkv_cache* c, const tkv_seq* seqs, const int32_t* nq, int32_t nseq, tkv_plan_info* out) {
  if (!c || !out) return TKV_E_INVAL;
  PlanSlot* s = nullptr;
  if (int rc = find_plan(c, seqs, nq, nseq, &s)) return rc;
  const Plan& P = s->plan;
  tkv_plan_info info{};
  info.groups = static_cast<int32_t>(P.groups.size());
  info.items = static_cast<int32_t>(P.items.size());
  info.block_entries = static_cast<int32_t>(P.blocks.size());
  info.unique_blocks = P.unique_blocks;
  info.unique_tokens = P.unique_tokens;
  info.partial_slots = P.partial_slots;
  for (int cls = 0; cls < kKernelClasses; ++cls) info.items_per_kernel[cls] = P.bucket_begin[cls + 1] - P.bucket_begin[cls];
  *out = info;
  return TKV_OK;
}

int tkv_set_option(tkv_cache* c, int32_t key, int64_t value) {
  if (!c) return TKV_E_INVAL;
  switch (key) {
    case TKV_OPT_TARGET_WGS:
      if (value < 1 || value > (1 << 24)) return TKV_E_RANGE;
      c->opt.target_wgs = static_cast<int32_t>(value);
      break;
    case TKV_OPT_MIN_CHUNK:
      if (value < 1 || value > (1 << 24)) return TKV_E_RANGE;
      c->opt.min_chunk = static_cast<int32_t>(value);
      break;
    case TKV_OPT_MAX_ROWS:
      if (value < 16 || value > kMaxRows) return TKV_E_RANGE;
      c->opt.max_rows = static_cast<int32_t>(value);
      break;
    case TKV_OPT_PLAN_CACHE:
      c->plan_cache = value != 0;
      break;
    case TKV_OPT_WAVES:
      if (value != 0 && value != 2 && value != 4 && value != 8) return TKV_E_RANGE;
      c->waves = static_cast<int32_t>(value);
      break;
    case TKV_OPT_CASCADE:
      if (value != 0 && value != 1) return TKV_E_RANGE;
      c->opt.cascade = static_cast<int32_t>(value);
      break;
    case TKV_OPT_CONCURRENT:
      if (value != 0 && value != 1) return TKV_E_RANGE;
      c->concurrent = static_cast<int32_t>(value);
      break;
    case TKV_OPT_PLAN_PATCH:
      if (value != 0 && value != 1) return TKV_E_RANGE;
      c->plan_patch = value != 0;
      break;
    case TKV_OPT_FUSED_NEW_TOKEN:
      if (value != 0 && value != 1) return TKV_E_RANGE;
      c->fuse_new = value != 0;
      break;
    default:
      return TKV_E_INVAL;
  }
  ++c->opt_epoch;
  return TKV_OK;
}

int tkv_get_option(const tkv_cache* c, int32_t key, int64_t* value) {
  if (!c || !value) return TKV_E_INVAL;
  switch (key) {
    case TKV_OPT_TARGET_WGS: *value = c->opt.target_wgs; break;
    case TKV_OPT_MIN_CHUNK: *value = c->opt.min_chunk; break;
    case TKV_OPT_MAX_ROWS: *value = c->opt.max_rows; break;
    case TKV_OPT_PLAN_CACHE: *value = c->plan_cache ? 1 : 0; break;
    case TKV_OPT_WAVES: *value = c->waves; break;
    case TKV_OPT_CASCADE: *value = c->opt.cascade; break;
    case TKV_OPT_CONCURRENT: *value = c->concurrent; break;
    case TKV_OPT_PLAN_PATCH: *value = c->plan_patch ? 1 : 0; break;
    case TKV_OPT_FUSED_NEW_TOKEN: *value = c->fuse_new ? 1 : 0; break;
    default: return TKV_E_INVAL;
  }
  return TKV_OK;
}

int tkv_profile_enable(tkv_cache* c, int32_t on) {
  if (!c) return TKV_E_INVAL;
  if (on && !c->has_pools) return TKV_E_NODEVICE;
  c->prof = on != 0;
  return TKV_OK;
}

int tkv_profile_read(tkv_cache* c, double* partial_ms, double* merge_ms, int64_t* calls) {
  if (!c) return TKV_E_INVAL;
  double pm = 0, mm = 0;
  int rc = TKV_OK;
  if (!c->prof_used.empty()) {
    DeviceGuard dg(c->device);
    for (auto& t : c->prof_used) {
      float a = 0.f, b = 0.f;
      if (hipEventSynchronize(t[2]) != hipSuccess || hipEventElapsedTime(&a, t[0], t[1]) != hipSuccess ||
          hipEventElapsedTime(&b, t[1], t[2]) != hipSuccess)
        rc = TKV_E_DEVICE;
      pm += a;
      mm += b;
      for (auto e : t) c->put_event(e);
    }
  }
  c->prof_used.clear();
  if (partial_ms) *partial_ms = pm;
  if (merge_ms) *merge_ms = mm;
  if (calls) *calls = c->prof_calls;
  c->prof_calls = 0;
  return rc;
}

}  // extern "C"
