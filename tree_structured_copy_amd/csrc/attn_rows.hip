// Tree attention for large query groups: K/V staged once in LDS for every row.
//
// When many queries share a prefix (the branches of a wide fork, the drafts of
// several speculative paths, the leaves under an MCTS node: the shared-ancestor
// case of the Dendrite article, "technical deep dive"), a group holds 3 to 16
// row tiles of 16 rows.  Holding all of them in one wave's registers (attn.hip)
// runs out of VGPRs, and giving each tile its own pass would re-read the prefix
// from HBM.  Here one workgroup streams the item's blocks through an LDS ring
// once, and its W waves each own TPW row tiles:
//   * every super-block (two consecutive blocks of the list) is copied from HBM
//     to LDS by all W waves together with global_load_lds_dwordx4 (direct to
//     LDS, no VGPRs), NS - 1 super-blocks ahead of the one being computed;
//   * the loads are issued from inline asm so that the waits are ours: the
//     compiler would otherwise wait for every outstanding LDS DMA at each
//     barrier and serialise the ring; one s_waitcnt vmcnt(N) + one barrier per
//     super-block keeps NS - 2 super-blocks in flight per wave besides the one
//     being read (the launcher picks NS: about two 16 KiB super-blocks in
//     flight per CU stream best);
//   * each wave reads the staged K and V fragments from LDS (conflict-free 16-B
//     lane-contiguous reads in the pool's MFMA operand order) and runs the same
//     S^T = K Q^T, online softmax and O^T += V^T P^T steps as attn.hip for each of
//     its tiles; a super-block no row of a wave can see is skipped by that wave;
//   * waves own disjoint rows, so no cross-wave merge is needed at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>

#include "attn_common.h"
#include "kernels.h"

namespace tkv {
namespace {

using namespace attn;

// TPW row tiles per wave; W waves per KV head; HPW KV heads per workgroup (the
// same item's block list for heads kvh0 .. kvh0 + HPW - 1: a group's heads see
// identical blocks); NS ring slots of one super-block (of every head).
// EARLY: a slot is refilled as soon as every wave has read its fragments (a
// second barrier per super-block), so all NS slots are in flight during the
// math; otherwise the refill waits for the next super-block's barrier and NS - 1
// are.  MINW: waves per SIMD the register budget must allow.
// An item's block list as staged in LDS: 16 bytes a block, the valid count
// sharing the id's word (ids are below kMaxPoolBlocks = 2^27), so the longest
// item (kRowsMaxItemBlocks) takes 16 KiB and two 64 KiB-ring workgroups still
// fit a CU's 160 KiB.
struct StagedBlock {
  uint32_t id_valid;  // id | valid << 27
  int32_t pos;
  uint64_t mask;
};
constexpr uint32_t kStagedIdMask = (1u << 27) - 1;

// X = NewTokens: the launch first writes a decode step's new tokens that lie
// in its items' blocks (write_new_tokens); X = NoNewTokens: it writes none.
template <class P, int D, int TPW, int W, int HPW, int NS, bool EARLY, int MINW, bool CAUSAL, class X>
__global__ __launch_bounds__(64 * W * HPW, MINW) void attn_rows_kernel(AttnArgs a, X x) {
  using E = typename P::elem;
  using F = typename P::template Frag<D>;
  constexpr int NDT = D / 16;
  constexpr int TILE_BYTES = 16 * D * static_cast<int>(sizeof(E));
  constexpr int LPT = TILE_BYTES / 1024;  // wave-loads per tile
  constexpr int HEAD_LOADS = 4 * LPT;     // K a, K b, V a, V b of one head
  constexpr int SB_LOADS = HPW * HEAD_LOADS;
  constexpr int LPW = rows_loads_per_wave<SB_LOADS, W * HPW>();
  constexpr int LOADERS = SB_LOADS / LPW;
  constexpr int STAGE = SB_LOADS * 1024;
  static_assert(NS >= 2 && (NS - 1) * LPW < 64, "ring depth");
  __shared__ __attribute__((aligned(1024))) char ring[NS * STAGE];
  // the item's block list: a.max_blocks entries, sized at launch
  extern __shared__ __attribute__((aligned(16))) char dyn_smem[];
  StagedBlock* ents = reinterpret_cast<StagedBlock*>(dyn_smem);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hsel = wave / W;     // which of the workgroup's heads this wave serves
  const int lw = wave - hsel * W;  // the wave's index among that head's waves
  const int g = lane >> 4, r = lane & 15;
  const int hgroups = a.hkv / HPW;
  const int kvh0 = (blockIdx.x % hgroups) * HPW;
  const int kvh = kvh0 + hsel;
  const DevItem it = a.items[a.item0 + blockIdx.x / hgroups];
  if constexpr (X::kActive) write_new_tokens<P, D, 64 * W * HPW, HPW>(x, it, kvh0, a.hkv, tid);
  const int nb = it.blk_count;
  const int nsb = (nb + 1) >> 1;
  const DevBlock* bl = a.blocks + it.blk_begin;
  const size_t tile_elems = 16 * D;
  const size_t bstride_bytes = static_cast<size_t>(a.hkv) * tile_elems * sizeof(E);
  const char* kbase = uniform_ptr(reinterpret_cast<const char*>(static_cast<const E*>(a.kpool) + kvh0 * tile_elems));
  const char* vbase = uniform_ptr(reinterpret_cast<const char*>(static_cast<const E*>(a.vpool) + kvh0 * tile_elems));
  const uint32_t ring_base = __builtin_amdgcn_readfirstlane(lds_byte_addr(ring));

  const int G = a.gsize;
  const int nrows = it.nq * G;

  // rows of this wave: tiles lw, lw + W, ... of head kvh; their query
  // indices load beside the ring's first block ids, so that the queries
  // themselves go out right behind the ring's first loads
  const uint64_t gmask = it.nq >= 64 ? ~0ull : ((1ull << it.nq) - 1);
  int qi[TPW], qj[TPW], qlim[TPW];
  uint64_t my_q = 0;  // group queries with a row in this wave's tiles
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tile = lw + W * t;
    const int R = 16 * tile + r;
    if (16 * tile < nrows) {
      const int j0 = (16 * tile) / G, j1 = min(nrows - 1, 16 * tile + 15) / G;
      for (int j = j0; j <= j1; ++j) my_q |= 1ull << j;
    }
    if (R < nrows) {
      const int j = R / G;
      qi[t] = a.gq[it.q_begin + j];
      qj[t] = j;
      qlim[t] = CAUSAL ? a.gqpos[it.q_begin + j] : 0;
    } else {
      qi[t] = -1;
      qj[t] = 0;
      qlim[t] = 0x7fffffff;
    }
  }

  // Issue this wave's share of super-block sp's loads into ring slot `slot`.
  // The ids of the first 64 blocks come straight from global memory, so the
  // ring's first super-blocks are in flight before the block list and the
  // queries are staged; later batches come from the staged list.
  int ib_base = 0, ib_id = lane < nb ? bl[lane].id : 0;  // ids of blocks [ib_base, ib_base + 64), one per lane
  // one wait for the ids, on every path, before the first ring load: a wait
  // the compiler placed at each (conditional) issue below would also drain
  // the super-blocks issued before it
  __builtin_amdgcn_s_waitcnt(0);
  auto issue = [&](int sp, int slot) {
    if (wave >= LOADERS) return;
    const int b0 = 2 * sp;
    if (b0 >= ib_base + 64) {
      ib_base = b0;
      ib_id = (b0 + lane < nb) ? static_cast<int>(ents[b0 + lane].id_valid & kStagedIdMask) : 0;
    }
    const int ida = __builtin_amdgcn_readlane(ib_id, b0 - ib_base);
    const int idb = (b0 + 1 < nb) ? __builtin_amdgcn_readlane(ib_id, b0 + 1 - ib_base) : ida;
#pragma unroll
    for (int k = 0; k < LPW; ++k) {
      const int i = wave * LPW + k;  // LDS slot i * 1024: head i / HEAD_LOADS, then K a, K b, V a, V b
      const int hh = i / HEAD_LOADS, j = i - hh * HEAD_LOADS;
      const int t = j / LPT, part = j - t * LPT;
      const char* src = ((t & 2) ? vbase : kbase) + static_cast<size_t>((t & 1) ? idb : ida) * bstride_bytes +
                        hh * TILE_BYTES;
      dma16(src, part * 1024 + lane * 16, ring_base + slot * STAGE + i * 1024);
    }
  };

  // The ring's first super-blocks.  Compiler-visible loads issued after them
  // make the compiler wait for them too where it waits for its own (the count
  // is in issue order); everything visible is complete before the loop below.
  constexpr int AHEAD = EARLY ? NS : NS - 1;  // super-blocks issued before the first is read
#pragma unroll
  for (int sp = 0; sp < AHEAD; ++sp)
    if (sp < nsb) issue(sp, sp);

  // the queries, right behind the ring's first loads
  F qf[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    if (qi[t] >= 0) {
      const int R = 16 * (lw + W * t) + r;
      const int h = kvh * G + (R - qj[t] * G);
      P::load_q(qf[t], static_cast<const E*>(a.q) + (static_cast<size_t>(qi[t]) * a.hq + h) * D, g);
    } else {
      P::zero(qf[t]);
    }
  }
  // the item's block list, staged once; waves read it 64 entries at a time
  // (lane k holds entry base + k) and take each super-block's fields with
  // v_readlane, so no LDS round trip sits on the per-super-block path
  for (int k = tid; k < nb; k += 64 * W * HPW) {
    const DevBlock e = bl[k];
    ents[k] = StagedBlock{static_cast<uint32_t>(e.id) | (static_cast<uint32_t>(e.valid) << 27), e.pos, e.mask};
  }

  float m[TPW], l[TPW];
  f32x4 acc[TPW][NDT];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    m[t] = kNegInf;
    l[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = a.scale_log2;
  const float tau_raw = kTau / sl2;  // the lazy-rescale threshold in raw score units
  const int min_lim = it.min_pos;
  const bool active = 16 * lw < nrows;

  // Every load the compiler can see (queries, group data, the block list) is
  // complete here, and it knows it, so it places no vmcnt waits of its own in
  // the loop below: those would also count our invisible ring loads and drain
  // the ring on every iteration.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // fields of blocks [cb_base, cb_base + 64), one per lane (zero past the list)
  int cb_base = -64, cb_valid = 0, cb_pos = 0;
  uint32_t cb_mlo = 0, cb_mhi = 0;
  for (int s = 0; s < nsb; ++s) {
    // super-block s has landed once this wave's loads of it are done (the
    // later AHEAD - 1 super-blocks may still be in flight) and every wave has
    // passed the barrier; without EARLY the barrier also frees slot (s - 1) % NS
    if (s + AHEAD <= nsb) wait_vm<(AHEAD - 1) * LPW>();
    else wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    if constexpr (!EARLY) {
      // (super-block NS - 1 went out with the prologue)
      if (s + NS - 1 < nsb) issue(s + NS - 1, (s + NS - 1) % NS);
    }

    const int b0 = 2 * s;
    if (b0 >= cb_base + 64) {
      cb_base = b0;
      const int k = b0 + lane;
      // selected by value, stored once (see the same refill in attn.hip)
      StagedBlock e{0, 0, 0};
      if (k < nb) e = ents[k];
      cb_valid = static_cast<int>(e.id_valid >> 27);
      cb_pos = e.pos;
      cb_mlo = static_cast<uint32_t>(e.mask);
      cb_mhi = static_cast<uint32_t>(e.mask >> 32);
    }
    const int la = b0 - cb_base;
    SBMeta e;
    e.va = __builtin_amdgcn_readlane(cb_valid, la);
    e.pa = __builtin_amdgcn_readlane(cb_pos, la);
    e.ma = (static_cast<uint64_t>(__builtin_amdgcn_readlane(cb_mhi, la)) << 32) |
           static_cast<uint32_t>(__builtin_amdgcn_readlane(cb_mlo, la));
    e.vb = __builtin_amdgcn_readlane(cb_valid, la + 1);
    e.pb = __builtin_amdgcn_readlane(cb_pos, la + 1);
    e.mb = (static_cast<uint64_t>(__builtin_amdgcn_readlane(cb_mhi, la + 1)) << 32) |
           static_cast<uint32_t>(__builtin_amdgcn_readlane(cb_mlo, la + 1));
    // refill slot s % NS with super-block s + NS once every wave is done with it
    auto refill_early = [&]() {
      if constexpr (EARLY) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        if (s + NS < nsb) issue(s + NS, s % NS);
      }
    };
    if (!active || ((e.ma | e.mb) & my_q) == 0) {
      refill_early();
      continue;
    }

    const uint32_t st = ring_base + (s % NS) * STAGE + hsel * 4 * TILE_BYTES;
    F ka, kb;
    typename P::template VPair<D> vp;
    P::load_tile_lds(ka, st + 0 * TILE_BYTES, lane);
    P::load_tile_lds(kb, st + 1 * TILE_BYTES, lane);
    const bool see_a = (e.ma & gmask) == gmask, see_b = (e.mb & gmask) == gmask;
    const bool need_mask = e.va < 16 || e.vb < 16 || !see_a || !see_b ||
                           (CAUSAL && (e.pa + 15 > min_lim || e.pb + 15 > min_lim));
    // all of this wave's scores first (the K fragments then die), V after
    float sc[TPW][8];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      // every tile of the wave runs (a tile past the group's rows has zero
      // queries and is never written): no per-tile branches to keep values across
      const f32x4 sa = P::qk(ka, qf[t]);
      const f32x4 sb = P::qk(kb, qf[t]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[t][i] = sa[i];
        sc[t][4 + i] = sb[i];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    P::template lds_vpair<D>(vp, st + 2 * TILE_BYTES, lane);
    refill_early();
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      // every tile of the wave runs (a tile past the group's rows has zero
      // queries and is never written): no per-tile branches to keep values across
      if (need_mask) {
        const bool qa = ((e.ma >> qj[t]) & 1ull) != 0, qb = ((e.mb >> qj[t]) & 1ull) != 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 4 * g + i;
          bool oka = tok < e.va && qa, okb = tok < e.vb && qb;
          if (CAUSAL) {
            oka = oka && (e.pa + tok <= qlim[t]);
            okb = okb && (e.pb + tok <= qlim[t]);
          }
          if (!oka) sc[t][i] = kNegInf;
          if (!okb) sc[t][4 + i] = kNegInf;
        }
      }
      // Lazy rescale: the row maximum is only formed (across the 4 lanes that
      // share a row) when some score of the wave exceeds its row's m by tau;
      // otherwise m stays and every weight is at most 2^tau.
      const float* x = sc[t];
      const float bm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      if (__any(bm > m[t] + tau_raw)) {
        float rm = fmaxf(bm, __shfl_xor(bm, 16));
        rm = fmaxf(rm, __shfl_xor(rm, 32));
        const float mn = fmaxf(m[t], rm);
        const float alpha = (m[t] == kNegInf) ? 0.f : fast_exp2((m[t] - mn) * sl2);
        l[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[t][dt] *= alpha;
        m[t] = mn;
      }
      // m is kept in raw score units; the exponent is (s - m) * log2(e) / sqrt(D),
      // the difference taken first so that the score equal to m weighs exactly 1
      const float mm = (m[t] == kNegInf) ? 0.f : m[t];
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = fast_exp2((x[i] - mm) * sl2);
      // the same expression on the lane's largest score: exactly its largest weight
      P::pv(vp, p, fast_exp2((bm - mm) * sl2), acc[t], l[t]);
      if constexpr (TPW > 1) __builtin_amdgcn_sched_barrier(0);  // one tile's weights live at a time
    }
  }
  // every DMA this wave issued must land before the workgroup's LDS is released
  wait_vm<0>();
  mfma_result_fence();

  // write this wave's rows: lane (g, r) holds O^T[16 dt + 4 g + i][row r]
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tile = lw + W * t;
    if (16 * tile >= nrows) break;
    float lt = l[t];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int R = 16 * tile + r;
    if (R >= nrows) continue;
    const int j = R / G;
    const int h = kvh * G + (R - j * G);
    if (it.part_base < 0) {
      const int qi = a.gq[it.q_begin + j];
      float* o = a.out + (static_cast<size_t>(qi) * a.hq + h) * D;
      // divided, not multiplied by 1 / l: a single visible key then gives its
      // value exactly, as the register kernel does
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4*>(o + 16 * dt + 4 * g) = acc[t][dt] / lt;
    } else if ((it.qmask >> j) & 1ull) {
      const size_t slot = static_cast<size_t>(it.part_base) + static_cast<size_t>(j) * a.hq + h;
      float* o = a.part_acc + slot * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(o + 16 * dt + 4 * g) = acc[t][dt];
      if (g == 0) {
        a.part_ml[2 * slot] = m[t];
        a.part_ml[2 * slot + 1] = lt;
      }
    }
  }
}

// Ring slots: as many super-blocks (of all the workgroup's heads) as fit in
// the LDS budget, at most 8.
template <class P, int D, int HPW, int BUDGET_KB>
constexpr int ring_slots() {
  constexpr int stage = HPW * 4 * 16 * D * static_cast<int>(sizeof(typename P::elem));
  return (BUDGET_KB * 1024 / stage) < 8 ? (BUDGET_KB * 1024 / stage) : 8;
}

template <class P, int D, int TPW, int W, int HPW, int NS, bool EARLY, int MINW, bool C, class X>
hipError_t launch_one(const AttnArgs& args, const X& x, int32_t n_items, hipStream_t s) {
  const size_t ents_bytes = sizeof(StagedBlock) * static_cast<size_t>(args.max_blocks > 0 ? args.max_blocks : 1);
  hipLaunchKernelGGL((attn_rows_kernel<P, D, TPW, W, HPW, NS, EARLY, MINW, C, X>), dim3(n_items * (args.hkv / HPW)),
                     dim3(64 * W * HPW), ents_bytes, s, args, x);
  char nm[112];
  snprintf(nm, sizeof nm, "attn_rows_kernel<%s, %d, %d, %d, %d, %d, %s, %d, %s%s>", P::kName, D, TPW, W, HPW, NS,
           EARLY ? "true" : "false", MINW, C ? "true" : "false", X::kActive ? ", NewTokens" : "");
  launch_log_add(nm);
  return hipGetLastError();
}

// Ring depth that keeps about 16 KiB of each workgroup's loads in flight
// beside the stage being read.  HBM serves these scattered tile streams best
// with about two 16 KiB stages in flight per CU: deeper rings measured slower
// (a 32-layer decode layer ran at 6.2 TB/s with four 16 KiB slots and two
// workgroups per CU, 6.8-7.0 TB/s with two).
template <class P, int D, int HPW>
constexpr int shallow_slots() {
  constexpr int stage = HPW * 4 * 16 * D * static_cast<int>(sizeof(typename P::elem));
  return 1 + (16384 / stage > 1 ? 16384 / stage : 1);
}

// Shapes by row tiles.  Up to 4 tiles: 4 waves and a 64 KiB ring, so two
// workgroups fit a CU; with no more workgroups than CUs the ring is filled
// deeper, as one workgroup then has the CU's loads in flight alone.  fp32 at
// d = 128 needs the registers of one workgroup per CU.
template <class P, int D, bool C, class X>
hipError_t launch_shape(int tiles, const AttnArgs& args, const X& x, int32_t n_items, hipStream_t s, int cus) {
  constexpr bool kSmall = kIsBF16<P> || D <= 64;
  if (tiles <= 4) {
    if constexpr (kSmall) {
      if (static_cast<int64_t>(n_items) * args.hkv > cus)
        return launch_one<P, D, 1, 4, 1, shallow_slots<P, D, 1>(), false, 2, C, X>(args, x, n_items, s);
      return launch_one<P, D, 1, 4, 1, ring_slots<P, D, 1, 64>(), false, 2, C, X>(args, x, n_items, s);
    } else {
      return launch_one<P, D, 1, 4, 1, ring_slots<P, D, 1, 128>(), false, 1, C, X>(args, x, n_items, s);
    }
  }
  if (tiles <= 6) {
    // two heads per workgroup where the head count allows, so that its 12 waves
    // spread evenly over the CU's four SIMDs (6 waves would sit 2, 2, 1, 1)
    if constexpr (kSmall) {
      if (args.hkv % 2 == 0) return launch_one<P, D, 1, 6, 2, shallow_slots<P, D, 2>(), false, 3, C, X>(args, x, n_items, s);
      return launch_one<P, D, 1, 6, 1, shallow_slots<P, D, 1>(), false, 3, C, X>(args, x, n_items, s);
    } else {
      return launch_one<P, D, 1, 6, 1, ring_slots<P, D, 1, 128>(), false, 2, C, X>(args, x, n_items, s);
    }
  }
  if (tiles <= 8) {
    if constexpr (kSmall) return launch_one<P, D, 1, 8, 1, shallow_slots<P, D, 1>(), false, 4, C, X>(args, x, n_items, s);
    else return launch_one<P, D, 1, 8, 1, ring_slots<P, D, 1, 128>(), false, 2, C, X>(args, x, n_items, s);
  }
  if (tiles <= 16) {
    if constexpr (kSmall) return launch_one<P, D, 1, 16, 1, shallow_slots<P, D, 1>(), false, 4, C, X>(args, x, n_items, s);
    else return launch_one<P, D, 2, 8, 1, ring_slots<P, D, 1, 128>(), false, 2, C, X>(args, x, n_items, s);
  }
  return hipErrorInvalidValue;
}

template <class P, int D>
hipError_t launch_c(int tiles, bool causal, const AttnArgs& args, const NewTokens* nt, int32_t n_items, hipStream_t s,
                    int cus) {
  if (nt)
    return causal ? launch_shape<P, D, true, NewTokens>(tiles, args, *nt, n_items, s, cus)
                  : launch_shape<P, D, false, NewTokens>(tiles, args, *nt, n_items, s, cus);
  return causal ? launch_shape<P, D, true, NoNewTokens>(tiles, args, NoNewTokens{}, n_items, s, cus)
                : launch_shape<P, D, false, NoNewTokens>(tiles, args, NoNewTokens{}, n_items, s, cus);
}

}  // namespace

hipError_t launch_attn_rows(int dtype, int head_dim, int tiles, bool causal, const AttnArgs& args, int32_t n_items,
                            hipStream_t stream, int cus, const NewTokens* nt) {
  if (n_items <= 0) return hipSuccess;
  if (dtype == 1 && head_dim == 128) return launch_c<BF16, 128>(tiles, causal, args, nt, n_items, stream, cus);
  if (dtype == 1 && head_dim == 64) return launch_c<BF16, 64>(tiles, causal, args, nt, n_items, stream, cus);
  if (dtype == 0 && head_dim == 128) return launch_c<F32, 128>(tiles, causal, args, nt, n_items, stream, cus);
  if (dtype == 0 && head_dim == 64) return launch_c<F32, 64>(tiles, causal, args, nt, n_items, stream, cus);
  return hipErrorInvalidValue;
}

}  // namespace tkv
