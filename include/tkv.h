/*
 * tkv -- attention over a forked, copy-on-write, block-table KV cache, for MI355X (gfx950).
 *
 * The method: the Dendrite article (ainews.cool, "Dendrite: O(1) KV cache forking",
 * section "technical deep dive") keeps the KV cache as a tree.  A prefix shared by
 * several branches is stored once; forking at position t copies nothing below t and
 * gives each branch new, empty leaves for the positions it will add; attention walks
 * the tree, taking keys and values from the shared ancestor path and then from the
 * branch's own leaf path.  The Dendrite demo tape ("the problem" section) names the
 * mechanism a copy-on-write block table.  The DSpark blog (second layer: predict,
 * verify in one parallel pass, accept or roll back) supplies the verification use:
 * a block of draft tokens is checked in one pass under a causal mask, and the
 * rejected tail is rolled back.
 *
 * This library keeps that tree on the host (nodes, refcounts, a lowest-free-id block
 * allocator; fork is O(n) in the number of children and O(1) in prefix length and
 * depth) and runs the attention on the GPU.  KV lives in caller-owned device pools,
 * in blocks of 16 token slots.
 *
 * Conventions for every entry point:
 *  - Return value: TKV_OK (0) or a negative tkv_status.  No exception crosses the ABI.
 *  - Host-side validation errors are returned before any state changes (strong
 *    guarantee): a failed call leaves the cache exactly as it was.
 *  - Device work is enqueued on the caller's stream (a hipStream_t passed as void*;
 *    NULL = the null stream) and is asynchronous: outputs are valid once the stream
 *    has reached the point of the call.  A failed launch is reported as TKV_E_DEVICE.
 *  - One cache is driven from one host thread and one stream.  Block reuse after a
 *    release is safe only because that stream orders the kernels that read and write
 *    a block.
 *  - Device pointers are plain device addresses; the library never frees caller
 *    memory.
 */
#ifndef TKV_H
#define TKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tkv_cache tkv_cache; /* opaque; the library owns the host metadata */

/* A sequence (branch) handle: (generation << 32) | slot.  0 is never a valid handle.
 * A released handle's generation is retired, so stale handles are detected. */
typedef uint64_t tkv_seq;

typedef enum { TKV_F32 = 0, TKV_BF16 = 1 } tkv_dtype;

typedef enum {
  TKV_OK = 0,
  TKV_E_INVAL = -1,     /* bad argument (n < 1, ntok < 1, bad config, NULL where required) */
  TKV_E_NOMEM = -2,     /* not enough free blocks (append is all-or-nothing) or host OOM */
  TKV_E_BADSEQ = -3,    /* handle was never issued or has been released */
  TKV_E_SHARED = -4,    /* truncation would remove tokens that other branches share */
  TKV_E_EMPTY = -5,     /* attention over a sequence with no tokens */
  TKV_E_RANGE = -6,     /* layer, length or query count out of range */
  TKV_E_DEVICE = -7,    /* a HIP call or kernel launch failed */
  TKV_E_WORKSPACE = -8, /* workspace too small (see tkv_workspace_size) */
  TKV_E_NODEVICE = -9   /* device call on a cache created without pools */
} tkv_status;

typedef struct tkv_config {
  int32_t num_layers;   /* >= 1 */
  int32_t num_q_heads;  /* multiple of num_kv_heads; q head h reads kv head h / (Hq/Hkv) */
  int32_t num_kv_heads; /* >= 1; Hq/Hkv <= 64 */
  int32_t head_dim;     /* 64 or 128 */
  int32_t block_size;   /* must be 16 */
  int32_t num_blocks;   /* blocks per layer in each pool, 1 .. 2^27 */
  int32_t dtype;        /* tkv_dtype of K, V and Q */
  int32_t reserved;     /* must be 0 */
  /* Caller-owned device pools, each num_layers * num_blocks * num_kv_heads * 16 *
   * head_dim elements of dtype, 16-byte aligned.  Both NULL = a host-only cache
   * (allocator and tables only; every device entry point returns TKV_E_NODEVICE).
   * Within a (layer, block, kv head) tile of 16 * head_dim elements the element
   * order is the library's own; only tkv_append writes it and tkv_gather reads it
   * back in token order. */
  void* k_pool;
  void* v_pool;
} tkv_config;

/* Create / destroy.  tkv_destroy frees host state only; pools stay the caller's.
 * The device that is current at tkv_create is the cache's device. */
int tkv_create(const tkv_config* cfg, tkv_cache** out);
int tkv_destroy(tkv_cache* c);

/* New empty root sequence. */
int tkv_seq_new(tkv_cache* c, tkv_seq* out);

/* Fork (article, "technical deep dive"): n >= 1 new handles that share every token
 * of `parent` by reference.  No block is allocated, written or copied, and no device
 * call is made; the cost is O(n), independent of the prefix length and of the tree
 * depth.  `parent` stays live.  Its current tail becomes read-only for everyone:
 * later appends on `parent` or on any child start a fresh block, so a partially
 * filled tail block at the fork point keeps its unused slots empty (at most 15).
 * out_children: host array of n handles, written only on success. */
int tkv_fork(tkv_cache* c, tkv_seq parent, int32_t n, tkv_seq* out_children);

/* Release a handle: a branch that lost is dropped (the article's case studies, AI
 * agent frameworks: several plans explored as branches, the one to keep chosen
 * afterwards; the DSpark blog, second layer: rejected draft paths discarded after
 * verification).  Blocks
 * no live handle can reach any more return to the free set.  The handle becomes
 * stale (TKV_E_BADSEQ afterwards).  Host only; no device call. */
int tkv_release(tkv_cache* c, tkv_seq s);

/* Append ntok >= 1 tokens to s (DSpark blog, third layer: each new token's K and V
 * are computed once and appended).  k, v: device arrays [num_layers][ntok][Hkv][head_dim]
 * of the cache dtype; they are read by kernels on `stream`.  Tokens fill the tail
 * block if it belongs to s alone, then fresh blocks (lowest free id first).
 * k = v = NULL reserves the slots without writing KV (metadata only; their KV
 * content is then undefined).  If the free blocks do not suffice, TKV_E_NOMEM and
 * nothing changes. */
int tkv_append(tkv_cache* c, tkv_seq s, int32_t ntok, const void* k, const void* v, void* stream);

/* Append ntok[i] >= 1 tokens to each of nseq >= 1 distinct handles seqs[i] in one
 * call (one kernel launch per 240 blocks written): the same as tkv_append on each
 * handle in batch order, with k, v device arrays [num_layers][sum ntok][Hkv][head_dim]
 * holding the handles' tokens one after another in batch order.  k = v = NULL
 * reserves the slots only.  All or nothing: a stale handle (TKV_E_BADSEQ), a count
 * < 1 or a handle given twice (TKV_E_INVAL), a total over 2^31 - 1 tokens
 * (TKV_E_RANGE) or too few free blocks for all of them (TKV_E_NOMEM) is found
 * before anything changes.  A decode loop appends its step's token to every
 * branch this way; appends that fit in the branches' last blocks leave the cached
 * plan of the next attention call valid up to an in-place update. */
int tkv_append_batch(tkv_cache* c, const tkv_seq* seqs, const int32_t* ntok, int32_t nseq,
                     const void* k, const void* v, void* stream);

/* Roll back s to new_len tokens (0 <= new_len <= length), e.g. to drop rejected
 * drafts after verification (DSpark blog, second layer: accept / roll back).  Only
 * tokens that s alone holds can be removed: if any position in [new_len, length) lies
 * in a block shared at some fork, TKV_E_SHARED and nothing changes.  new_len ==
 * length is a no-op.  Freed blocks return to the free set. */
int tkv_truncate(tkv_cache* c, tkv_seq s, int64_t new_len);

/* Device workspace needed by an attention call with these arguments (nq = NULL for
 * decode).  Builds (and caches) the call's plan.  *bytes may be 0.  nseq >= 1 (an
 * empty batch is TKV_E_INVAL here and in the attention calls).  It takes the
 * handles, not just their count and the query total, because the workspace holds
 * the split-K partial records, whose number depends on how the batch's paths
 * overlap and how long they are: the same (nseq, total queries) needs none for a
 * batch of long independent paths cut one item per group and megabytes for a
 * search tree cut into many chunks. */
int tkv_workspace_size(tkv_cache* c, const tkv_seq* seqs, const int32_t* nq, int32_t nseq,
                       size_t* bytes);

/* Decode attention (article, "technical deep dive": attention traverses the tree,
 * gathering K and V from the shared ancestor path and the branch's leaf path).  For
 * each handle i and query head h, with L_i tokens on its path and g = h / (Hq/Hkv):
 *   out[i][h] = sum_j softmax_j(q[i][h] . K_i[j][g] / sqrt(head_dim)) V_i[j][g],  j < L_i
 * q: device [nseq][Hq][head_dim] in the cache dtype; out: device fp32 [nseq][Hq][head_dim].
 * ws: device scratch of at least tkv_workspace_size() bytes (may be NULL if that is 0),
 * owned by the call until the stream passes it.  A handle may appear more than once.
 * Ordering: the call's work is ordered on `stream`; when its plan holds several kernel
 * classes, they run one after another on `stream`, or at once on side streams of the
 * library's own (default priority) forked from and joined back to `stream` with events
 * (TKV_OPT_CONCURRENT), so everything the call does is complete once `stream` passes
 * the point where the call was made.
 * TKV_E_EMPTY if a handle has no tokens. */
int tkv_attend_decode(tkv_cache* c, int32_t layer, const tkv_seq* seqs, int32_t nseq,
                      const void* q, float* out, void* ws, size_t ws_bytes, void* stream);

/* One layer of a decode step whose new token is written by the call (fused append
 * + decode, in the generation loop of the article's fork-based decoding): for each
 * handle i (each at most once), its last token -- which must lie in the handle's
 * own tip node, e.g. reserved for all layers by tkv_append_batch with k = v = NULL
 * -- gets K = k_new[i], V = v_new[i] for `layer` (device [nseq][Hkv][head_dim], cache
 * dtype), then the call is tkv_attend_decode over the paths that include it.  With up
 * to 192 handles, and no change to the cached plan since its last use other than
 * these tokens (the usual decode step after tkv_append_batch reserved them), the
 * attention launch itself writes each token -- the workgroup that reads its block
 * writes it first -- and the block's valid count in the plan: one launch per step
 * (TKV_OPT_FUSED_NEW_TOKEN).  Otherwise a preparation launch (one per 128 tokens)
 * writes them and the plan's changed words before the attention kernels, on
 * `stream`.  A token that opened its block is written with zeros in the block's
 * other slots.  Errors as
 * tkv_attend_decode, plus TKV_E_INVAL for a handle given twice or a null k_new /
 * v_new, and TKV_E_SHARED when a handle's last token is shared with other branches
 * (its tip node was forked, or it has no tokens of its own). */
int tkv_attend_decode_new_token(tkv_cache* c, int32_t layer, const tkv_seq* seqs, int32_t nseq,
                                const void* k_new, const void* v_new, const void* q, float* out,
                                void* ws, size_t ws_bytes, void* stream);

/* As tkv_attend_decode_new_token, with ntok[i] new tokens for handle i (1 <= ntok[i]
 * <= 16): its last ntok[i] tokens, which must all lie in its last block and its own tip
 * node -- e.g. a node of ntok[i] tokens reserved for every layer by tkv_append_batch
 * with k = v = NULL after a fork, as a tree search expands a node (Dendrite demo tape,
 * "MCTS demo": each expansion forks and extends the children before evaluating them).
 * Their K and V for `layer` are rows [r_i, r_i + ntok[i]) of k_new / v_new (device
 * [sum ntok][Hkv][head_dim], cache dtype), r_i = ntok[0] + ... + ntok[i-1].  One launch
 * per call under the same conditions as tkv_attend_decode_new_token (the records are
 * per tail block: a node opened by the tokens is written whole, zeros after them).
 * TKV_E_RANGE if some ntok[i] is outside 1..16 or the tokens would reach into an
 * earlier block; otherwise errors as tkv_attend_decode_new_token. */
int tkv_attend_decode_new_tokens(tkv_cache* c, int32_t layer, const tkv_seq* seqs, const int32_t* ntok,
                                 int32_t nseq, const void* k_new, const void* v_new, const void* q,
                                 float* out, void* ws, size_t ws_bytes, void* stream);

/* tkv_attend_verify whose verified tokens are new: handle i's last nq[i] tokens
 * (1 <= nq[i] <= 16), which must all lie in its last block and its own tip node --
 * the draft tokens of a speculative step, reserved for every layer by
 * tkv_append_batch with k = v = NULL after the fork into draft paths -- get their K
 * and V for `layer` from rows [r_i, r_i + nq[i]) of k_new / v_new (device
 * [sum nq][Hkv][head_dim], cache dtype), r_i = nq[0] + ... + nq[i-1], and are
 * verified in the same call: the target model computes each layer's K/V for the
 * drafts in the pass that verifies them, and they stay in the cache for the
 * accepted ones (DSpark blog, second layer: verify the drafts in parallel; third
 * layer: each token's K/V is computed once and kept).  One launch per call under the
 * conditions of tkv_attend_decode_new_token (at most 192 handles, the cached plan
 * changed only by these tokens); otherwise a preparation launch writes them first.
 * Errors as tkv_attend_verify and tkv_attend_decode_new_tokens. */
int tkv_attend_verify_new_tokens(tkv_cache* c, int32_t layer, const tkv_seq* seqs, const int32_t* nq, int32_t nseq,
                                 const void* k_new, const void* v_new, const void* q, float* out, void* ws,
                                 size_t ws_bytes, void* stream);

/* tkv_attend_decode for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same plan and kernels as tkv_attend_decode, with the plan and the split-K
 * partial records in a fixed workspace the library holds on each device (a
 * file-scope device array of 64 MiB, present from the first tkv_create on that
 * device until the process ends), so no workspace argument is taken.  The plan
 * is uploaded from a pinned staging buffer of 4 MiB made for it at tkv_create
 * (never grown; other calls use staging of their own).  The call
 * makes no hipMalloc, hipFree, host-pinned allocation, stream or event.
 * TKV_E_WORKSPACE if the plan and its partial records exceed the fixed
 * workspace or the plan exceeds the staging; otherwise errors as
 * tkv_attend_decode.  Every call on one GPU shares that GPU's workspace: calls
 * that overlap on the device (different streams, or different caches, without
 * ordering between them) race.  The profiling events are not recorded for it. */
int tkv_attend_decode_noalloc(tkv_cache* c, int32_t layer, const tkv_seq* seqs, int32_t nseq,
                              const void* q, float* out, void* stream);

/* Verification attention (DSpark blog, second layer: a block of drafts checked in one
 * parallel pass).  The last nq[i] tokens of handle i (1 <= nq[i] <= L_i) are queries;
 * the query at absolute position p attends over positions 0..p of its own path.
 * With one handle per draft path (forked from the shared prefix) this is the
 * tree-causal mask over prefix plus the path's own earlier drafts.
 * q: device [sum nq][Hq][head_dim], rows ordered by handle then position;
 * out: device fp32, same shape. */
int tkv_attend_verify(tkv_cache* c, int32_t layer, const tkv_seq* seqs, const int32_t* nq,
                      int32_t nseq, const void* q, float* out, void* ws, size_t ws_bytes,
                      void* stream);

/* Copy one layer of s's K and V history, in token order, to device arrays
 * k_out, v_out [length][Hkv][head_dim] (cache dtype).  For checking what
 * tkv_append stored. */
int tkv_gather(tkv_cache* c, tkv_seq s, int32_t layer, void* k_out, void* v_out, void* stream);

/* ---- introspection (host only, no device calls) ---- */
int tkv_seq_len(const tkv_cache* c, tkv_seq s, int64_t* len);
/* s's block table, root first: ids[i] and valid[i] (slots in use) for i < *n.
 * cap = capacity of ids/valid; if cap < needed, *n = needed and TKV_E_RANGE. */
int tkv_block_table(const tkv_cache* c, tkv_seq s, int32_t* ids, int32_t* valid, int32_t cap,
                    int32_t* n);
/* Number of live handles whose table holds the block (0 = free). */
int tkv_block_refcount(const tkv_cache* c, int32_t block, int32_t* rc);
/* Same for every block at once: rc[num_blocks]. */
int tkv_block_refcounts(const tkv_cache* c, int32_t* rc);
int tkv_num_free(const tkv_cache* c, int32_t* n);

typedef struct tkv_counters {
  int64_t blocks_taken;       /* blocks moved from the free set into use */
  int64_t blocks_freed;
  int64_t nodes_created;
  int64_t nodes_freed;
  int64_t block_ids_copied;   /* block-table entries copied by any operation (fork: none) */
  int64_t plans_built;
  int64_t plans_uploaded;     /* whole plans copied to the device */
  int64_t plans_patched;      /* device copies updated in place instead of uploaded whole (TKV_OPT_PLAN_PATCH):
                                 after appends inside tip blocks, and plans_reused */
  int64_t plans_reused;       /* plans built for a new batch that took over the device copy of a cached plan
                                 of the same shape differing only in block ids (the next attention launch
                                 rewrites those ids); also counted in plans_built and plans_patched */
} tkv_counters;
int tkv_get_counters(const tkv_cache* c, tkv_counters* out);

/* Names of the kernels the last attention call on c launched, in launch order,
 * "name<template arguments>" joined by ';' (e.g. the attention kernel and the
 * merge), NUL-terminated into buf[cap].  TKV_E_RANGE if cap is too small (buf
 * then holds as much as fits).  For naming measured kernels. */
int tkv_last_kernels(const tkv_cache* c, char* buf, int32_t cap);

/* Shape of the plan an attention call with these arguments uses (builds it). */
typedef struct tkv_plan_info {
  int32_t groups;          /* query groups (<= TKV_OPT_MAX_ROWS rows each, one KV pass per group) */
  int32_t items;           /* work items; one workgroup per item and KV head */
  int32_t block_entries;   /* block visits summed over groups */
  int32_t unique_blocks;   /* distinct blocks the call reads */
  int64_t unique_tokens;   /* valid token slots in those blocks */
  int64_t partial_slots;   /* fp32 partial records in the workspace */
  int32_t items_per_kernel[6]; /* items run by each kernel shape: groups of 1, 2, 3-4, 5-6, 7-8, 9-16 row tiles */
} tkv_plan_info;
int tkv_plan_info_get(tkv_cache* c, const tkv_seq* seqs, const int32_t* nq, int32_t nseq,
                      tkv_plan_info* out);

/* ---- tuning knobs (keys) ---- */
enum {
  TKV_OPT_TARGET_WGS = 1,   /* workgroups an attention call aims for (default: the device's CU count) */
  TKV_OPT_MIN_CHUNK = 2,    /* fewest blocks per split-K work item (default 32; a quarter of it for
                               groups of 3+ row tiles); a call too small to fill the GPU at that
                               size is cut into items of at least 4 blocks instead */
  TKV_OPT_MAX_ROWS = 3,     /* max rows (queries x Hq/Hkv) per group: 16..256 (default 128) */
  TKV_OPT_PLAN_CACHE = 4,   /* 1 = reuse uploaded plans while the tree is unchanged (default) */
  TKV_OPT_WAVES = 5,        /* waves per one/two-tile workgroup: 2, 4 or 8 (0 = by launch size) */
  TKV_OPT_CASCADE = 6,      /* 1 = a group of 8+ row tiles hands blocks that only one row tile's
                               queries see to one-tile subgroups, merged after; 0 = off (default) */
  TKV_OPT_CONCURRENT = 7,   /* how a call's kernel classes run: 0 = one after another on the call's
                               stream (default); 1 = at once, on side streams of the library's own
                               forked from and joined back to the call's stream */
  TKV_OPT_PLAN_PATCH = 8,   /* 1 = a cached plan made before appends that each fitted in their tip
                               node's last block (no new block, node, fork, release or truncation
                               since) is updated in place: the changed block counts and query
                               positions are written into its device copy by a small kernel
                               (default); 0 = such a plan is rebuilt and uploaded whole */
  TKV_OPT_FUSED_NEW_TOKEN = 9 /* 1 = tkv_attend_decode_new_token(s) writes its tokens (and their blocks'
                               valid counts in the plan) from the attention launch itself when it
                               can: one launch per step (default); 0 = always by a preparation
                               launch first */
};
int tkv_set_option(tkv_cache* c, int32_t key, int64_t value);
int tkv_get_option(const tkv_cache* c, int32_t key, int64_t* value);

/* ---- profiling: HIP events around the attention kernels, on the call's stream ---- */
int tkv_profile_enable(tkv_cache* c, int32_t on);
/* Waits for the recorded events, returns the summed milliseconds of the partial
 * (attention) kernels and of the merge kernel and the number of attention calls
 * since the last read, then resets. */
int tkv_profile_read(tkv_cache* c, double* partial_ms, double* merge_ms, int64_t* calls);

const char* tkv_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* TKV_H */
