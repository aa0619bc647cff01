// Tree attention kernels for gfx950.
//
// Dendrite article (ainews.cool, "technical deep dive"): a branch's query
// attends over the keys and values of its shared ancestor path and then of its
// own leaf path.  The planner has cut the batch into groups of at most 128 rows
// by default, 256 at most (rows = the group's queries x the query heads that
// share one KV head) and
// lists each group's blocks once, with a mask of which queries see each block.
//
// One workgroup (W = 2, 4 or 8 waves) runs one work item (a run of a group's
// block list) for one KV head.  Each wave takes a contiguous share of the
// item's super-blocks (two blocks each) and keeps, for all of the group's rows, a
// flash-decoding state (running max m, sum l, output accumulator) in
// registers:
//   * a block's K tile arrives with four contiguous 1 KiB wave loads already in
//     MFMA operand order (layout.h) and S^T = K Q^T for 16 tokens x 16 rows is a
//     handful of MFMAs: every key is fetched from HBM once per group, however
//     many sibling branches and GQA heads read it;
//   * the S^T fragment a lane gets (4 tokens of one row) is exactly the operand
//     P^T the P.V MFMA needs, so the softmax stays in registers;
//   * the running max is rescaled lazily (only when it grows by more than 2^8,
//     which bounds every weight by 2^8 and keeps fp32 sums exact enough).
// At the end the W waves' states are merged through LDS; an item that covers its
// whole group writes normalised outputs, otherwise it writes fp32 partials
// (m, l, acc) and attn_merge combines them (log-sum-exp, exp2 domain).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cstdio>

#include "attn_common.h"
#include "kernels.h"

namespace tkv {
namespace {

using namespace attn;

// X = NewTokens: the launch also writes a decode step's new tokens that lie
// in its items' blocks, each by the wave that reads it, before reading it;
// X = NoNewTokens: it writes none.
template <class P, int D, int T, int W, bool CAUSAL, class X>
__global__ __launch_bounds__(64 * W) void attn_partial_kernel(AttnArgs a, X x) {
  using E = typename P::elem;
  using F = typename P::template Frag<D>;
  constexpr int NDT = D / 16;
  constexpr int NT = 64 * W;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int kvh = blockIdx.x % a.hkv;
  const DevItem it = a.items[a.item0 + blockIdx.x / a.hkv];
  const int nb = it.blk_count;
  const int nsb = (nb + 1) >> 1;
  // super-blocks of this wave: a contiguous share of the item (two waves
  // streaming far-apart halves measured about 1 % faster than alternating)
  const int per_w = (nsb + W - 1) / W, start_w = wave * per_w;
  const int nmine = nsb > start_w ? min(per_w, nsb - start_w) : 0;
  const DevBlock* bl = a.blocks + it.blk_begin;
  const size_t tile = 16 * D;
  const size_t bstride = static_cast<size_t>(a.hkv) * tile;
  const E* kbase = static_cast<const E*>(a.kpool) + static_cast<size_t>(kvh) * tile;
  const E* vbase = static_cast<const E*>(a.vpool) + static_cast<size_t>(kvh) * tile;

  // Block-list entries of this wave, one per lane, 32 super-blocks per batch:
  // lane j holds block 2 * (start_w + 32 * batch + j / 2) + j % 2.  Reading
  // them with readlane keeps scalar-load latency out of the streaming loop.
  int e_id = -1, e_valid = 0, e_pos = 0;
  uint32_t e_mlo = 0, e_mhi = 0;
  int cur_batch = -1;
  // X = NewTokens: the item's new-token records (tail blocks [tk0, tk0 + tkc),
  // at most 64); each wave keeps their (entry, valid count) pairs in LDS.
  // When some record of the launch holds several tokens (a node the step
  // opens: whole tiles), the whole workgroup writes the item's records first,
  // before anything is loaded, and the owning waves write none.
  if constexpr (X::kActive) {
    if (x.multi) write_new_tokens<P, D, NT, 1>(x, it, kvh, a.hkv, tid);
  }
  const int tk0 = X::kActive ? (it.tails & 0xffff) : 0;
  const int tkc = [&]() {
    if constexpr (X::kActive) return x.multi ? 0 : (it.tails >> 16);
    else return 0;
  }();
  __shared__ int2 s_tok[X::kActive ? W : 1][X::kActive ? 64 : 1];
  bool tk_loaded = false;
  // X = NewTokens with id patches: the (entry, id) pairs of this item, in LDS
  // (the same list for every wave)
  __shared__ int2 s_ids[X::kActive ? kMaxIdPatches : 1];
  int nids = 0;
  auto correct_id = [&]() {
    if constexpr (X::kActive) {
      if (nids == 0 || cur_batch < 0) return;
      const int b = 2 * (start_w + 32 * cur_batch + (lane >> 1)) + (lane & 1);
      for (int i = 0; i < nids; ++i) {
        const int2 ei = s_ids[i];
        if (ei.x == it.blk_begin + b && e_id >= 0) e_id = ei.y;
      }
    }
  };
  // a block this launch writes a new token into holds one more token than the
  // plan's copy may say: the valid counts of the loaded batch, corrected
  auto correct_valid = [&]() {
    if constexpr (X::kActive) {
      if (!tk_loaded || cur_batch < 0) return;
      const int b = 2 * (start_w + 32 * cur_batch + (lane >> 1)) + (lane & 1);
      for (int i = 0; i < tkc; ++i) {
        const int2 ev = s_tok[wave][i];
        if (ev.x >= 0 && ev.x == it.blk_begin + b) e_valid = ev.y;
      }
    }
  };
  // (the entry is selected by value and stored once: branches that each store
  // the fields let the compiler merge their last stores through a selected
  // pointer, which puts these registers on the stack)
  auto load_entries = [&](int batch) {
    const int sbk = 32 * batch + (lane >> 1);
    const int b = 2 * (start_w + sbk) + (lane & 1);
    DevBlock e{-1, 0, 0, 0, 0};
    if (sbk < nmine && b < nb) e = bl[b];
    e_id = e.id;
    e_valid = e.valid;
    e_pos = e.pos;
    e_mlo = static_cast<uint32_t>(e.mask);
    e_mhi = static_cast<uint32_t>(e.mask >> 32);
    cur_batch = batch;
    correct_valid();
    correct_id();
  };
  auto meta = [&](int k) {
    if ((k >> 5) != cur_batch) load_entries(k >> 5);
    const int ja = 2 * (k & 31), jb = ja + 1;
    SBMeta m;
    m.ida = __builtin_amdgcn_readlane(e_id, ja);
    m.idb = __builtin_amdgcn_readlane(e_id, jb);
    m.va = __builtin_amdgcn_readlane(e_valid, ja);
    m.vb = __builtin_amdgcn_readlane(e_valid, jb);
    m.pa = __builtin_amdgcn_readlane(e_pos, ja);
    m.pb = __builtin_amdgcn_readlane(e_pos, jb);
    m.ma = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(e_mhi, ja))) << 32) |
           static_cast<uint32_t>(__builtin_amdgcn_readlane(e_mlo, ja));
    m.mb = (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(e_mhi, jb))) << 32) |
           static_cast<uint32_t>(__builtin_amdgcn_readlane(e_mlo, jb));
    if (m.idb < 0) {  // odd tail: reload block a, fully masked
      m.idb = m.ida;
      m.vb = 0;
    }
    return m;
  };
  using VP = typename P::template VPair<D>;
  auto load_sb = [&](F& ka, F& kb, VP& v, const SBMeta& m) {
    P::load_tile(ka, kbase + static_cast<size_t>(m.ida) * bstride, lane);
    P::load_tile(kb, kbase + static_cast<size_t>(m.idb) * bstride, lane);
    P::load_vpair(v, vbase + static_cast<size_t>(m.ida) * bstride, vbase + static_cast<size_t>(m.idb) * bstride,
                  lane);
  };

  F kA0, kA1, kB0, kB1;
  VP vA, vB;
  SBMeta mA, mB;
  // A decode step's new tokens in this wave's blocks are written by the wave
  // itself.  The first super-block's loads go out first; then the item's
  // token records (one load per lane), the values of the wave's tokens and
  // their stores.  If the first super-block holds a written block it is loaded
  // again once the stores have landed; otherwise the wave waits for them
  // before loading its first super-block that holds one.
  if constexpr (X::kActive) {
    if (x.nid > 0) {
      // a reused plan's new block ids: this item's are written into the plan
      // (every KV head's workgroup writes the same values) and read from LDS
      // wherever the old ids were loaded; the first loads wait for them
      IdPatch pch{-1, 0};
      if (lane < x.nid) pch = x.ids[lane];
      const bool mine = pch.entry >= it.blk_begin && pch.entry < it.blk_begin + nb;
      const uint64_t m = __ballot(mine);
      nids = __popcll(m);
      if (mine) {
        const int k = __popcll(m & ((1ull << lane) - 1));
        if (wave == 0) {
          s_ids[k] = int2{pch.entry, pch.id};
          __builtin_nontemporal_store(pch.id, &x.blocks[pch.entry].id);
        }
      }
      __syncthreads();
      correct_id();
    }
  }
  if (nmine > 0) {
    mA = meta(0);
    load_sb(kA0, kA1, vA, mA);
  }
  int tok_sb = 0x7fffffff;  // index in this wave's share of its first super-block that gets a token
  if constexpr (X::kActive) {
    using TU = TokUnits<P, D>;
    if (tkc > 0) {
      int tk_entry = -1, tk_blk = 0, tk_slot = 0, tk_n = 0, tk_src = 0;
      if (lane < tkc) {
        // records past x.n are not this launch's (a launch with id patches
        // and no tokens lists none)
        NewTok t{-1, 0, 0, 0, 0};
        if (tk0 + lane < x.n) t = x.tok[tk0 + lane];
        tk_entry = t.entry;
        tk_blk = t.blk;
        tk_slot = t.slot;
        tk_n = t.n;
        tk_src = t.src;
        s_tok[wave][lane] = int2{t.entry, t.slot + t.n};
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS writes done (a wave reads only its own)
      tk_loaded = true;
      correct_valid();
      if (nmine > 0) mA = meta(0);
      const int my_lo = it.blk_begin + 2 * start_w, my_hi = it.blk_begin + 2 * (start_w + nmine);
      const bool own = tk_entry >= my_lo && tk_entry < my_hi;
      uint64_t mine = __ballot(own);
      if (mine) {
        const int first = __builtin_ctzll(mine);
        tok_sb = ((__builtin_amdgcn_readlane(tk_entry, first) - it.blk_begin) >> 1) - start_w;
        auto rec = [&](int i) {
          return NewTok{__builtin_amdgcn_readlane(tk_entry, i), __builtin_amdgcn_readlane(tk_blk, i),
                        static_cast<int16_t>(__builtin_amdgcn_readlane(tk_slot, i)),
                        static_cast<int16_t>(__builtin_amdgcn_readlane(tk_n, i)), __builtin_amdgcn_readlane(tk_src, i)};
        };
        // records that open their block (rare in a decode step: whole tiles)
        // and records of several tokens in a block that has others, one at a
        // time; then single tokens, a few at a time with all their values'
        // loads in flight together
        uint64_t fresh = __ballot(own && (tk_slot == 0 || tk_n > 1));
        while (fresh) {
          const NewTok t = rec(__builtin_ctzll(fresh));
          fresh &= fresh - 1;
          const int nu = TU::units(t);
          for (int u0 = lane; u0 < nu; u0 += 4 * 64) {
            u32x4 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (u0 + 64 * k < nu) v[k] = TU::value(x, t, kvh, a.hkv, u0 + 64 * k);
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (u0 + 64 * k < nu) TU::store(x, t, kvh, a.hkv, u0 + 64 * k, v[k]);
          }
          if (lane == 0) x.blocks[t.entry].valid = t.slot + t.n;
        }
        uint64_t plain = __ballot(own && tk_slot != 0 && tk_n == 1);
        constexpr int RPT = (TU::kPlain + 63) / 64;  // 64-unit rows per token
        constexpr int MAXT = 4;                      // tokens whose values are in flight at once
        while (plain) {
          NewTok t[MAXT];
          int nt = 0;
#pragma unroll
          for (int j = 0; j < MAXT; ++j) {
            t[j] = NewTok{-1, 0, 0, 0, 0};
            if (plain) {
              t[j] = rec(__builtin_ctzll(plain));
              plain &= plain - 1;
              nt = j + 1;
            }
          }
          u32x4 v[MAXT][RPT];
#pragma unroll
          for (int j = 0; j < MAXT; ++j) {
            if (j >= nt) break;
#pragma unroll
            for (int rr = 0; rr < RPT; ++rr)
              if (rr * 64 + lane < TU::kPlain) v[j][rr] = TU::value(x, t[j], kvh, a.hkv, rr * 64 + lane);
          }
          // the values, and the first super-block issued before them, have
          // landed: the stores then go out after every load the loop's first
          // step needs, so nothing waits for their acknowledgement until the
          // super-block that reads them
          __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
          for (int j = 0; j < MAXT; ++j) {
            if (j >= nt) break;
#pragma unroll
            for (int rr = 0; rr < RPT; ++rr)
              if (rr * 64 + lane < TU::kPlain) TU::store(x, t[j], kvh, a.hkv, rr * 64 + lane, v[j][rr]);
            if (lane == 0) x.blocks[t[j].entry].valid = t[j].slot + t[j].n;
          }
        }
        if (tok_sb == 0) {
          __builtin_amdgcn_s_waitcnt(0);
          load_sb(kA0, kA1, vA, mA);
        }
      }
    }
  }

  // queries: row R = 16 t + r of the group is query R / G, head kvh * G + R % G
  const int G = a.gsize;
  const int nrows = it.nq * G;
  const uint64_t gmask = it.nq >= 64 ? ~0ull : ((1ull << it.nq) - 1);
  F qf[T];
  int qj[T], qlim[T], qix[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const int R = 16 * t + r;
    if (R < nrows) {
      const int j = R / G;
      const int h = kvh * G + (R - j * G);
      const int qi = a.gq[it.q_begin + j];
      P::load_q(qf[t], static_cast<const E*>(a.q) + (static_cast<size_t>(qi) * a.hq + h) * D, g);
      qj[t] = j;
      qix[t] = qi;
      qlim[t] = CAUSAL ? a.gqpos[it.q_begin + j] : 0;
    } else {
      P::zero(qf[t]);
      qj[t] = 0;
      qix[t] = 0;
      qlim[t] = 0x7fffffff;
    }
  }

  float m[T], l[T];
  f32x4 acc[T][NDT];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    m[t] = kNegInf;
    l[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[t][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sl2 = a.scale_log2;
  const float tau_raw = kTau / sl2;  // the lazy-rescale threshold in raw score units
  const int min_lim = it.min_pos;

  auto process = [&](const F& ka, const F& kb, const VP& v, const SBMeta& e) {
    const bool see_a = (e.ma & gmask) == gmask, see_b = (e.mb & gmask) == gmask;
    const bool need_mask = e.va < 16 || e.vb < 16 || !see_a || !see_b || (CAUSAL && e.pb + 15 > min_lim) ||
                           (CAUSAL && e.pa + 15 > min_lim);
#pragma unroll
    for (int t = 0; t < T; ++t) {
      const f32x4 sa = P::qk(ka, qf[t]);
      const f32x4 sb = P::qk(kb, qf[t]);
      float sc[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[i] = sa[i];
        sc[4 + i] = sb[i];
      }
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
          if (!oka) sc[i] = kNegInf;
          if (!okb) sc[4 + i] = kNegInf;
        }
      }
      // Lazy rescale: the row maximum is only formed (across the 4 lanes that
      // share a row) when some score of the wave exceeds its row's m by tau;
      // otherwise m stays and every weight is at most 2^tau.
      const float bm =
          fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
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
      for (int i = 0; i < 8; ++i) p[i] = fast_exp2((sc[i] - mm) * sl2);
      // the same expression on the lane's largest score: exactly its largest weight
      P::pv(v, p, fast_exp2((bm - mm) * sl2), acc[t], l[t]);
    }
  };

  if (nmine > 0) {
    for (int k = 0; k < nmine; k += 2) {
      mB = meta(min(k + 1, nmine - 1));
      if constexpr (X::kActive) {
        if (k + 1 == tok_sb) __builtin_amdgcn_s_waitcnt(0);
      }
      load_sb(kB0, kB1, vB, mB);
      process(kA0, kA1, vA, mA);
      if (k + 1 >= nmine) break;
      mA = meta(min(k + 2, nmine - 1));
      if constexpr (X::kActive) {
        if (k + 2 == tok_sb) __builtin_amdgcn_s_waitcnt(0);
      }
      load_sb(kA0, kA1, vA, mA);
      process(kB0, kB1, vB, mB);
    }
  }

  mfma_result_fence();
#pragma unroll
  for (int t = 0; t < T; ++t) {
    l[t] += __shfl_xor(l[t], 16);
    l[t] += __shfl_xor(l[t], 32);
  }

  // merge the W waves' states through LDS, one row tile at a time: each wave
  // puts its rows there row-major (16-byte runs, as the MFMA leaves them),
  // then every thread finishes four consecutive elements of a row at a time,
  // the row's maximum and wave weights formed once per piece, so that a
  // wave's stores cover whole rows
  constexpr int RS = D + 4;  // LDS row stride in floats
  constexpr int P4 = D / 4;  // four-element pieces per row
  __shared__ float s_m[W][16];
  __shared__ float s_l[W][16];
  __shared__ int s_qi[16];
  __shared__ __attribute__((aligned(16))) float s_acc[W][16][RS];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    if (16 * t >= nrows) break;
    if (g == 0) {
      s_m[wave][r] = m[t];
      s_l[wave][r] = l[t];
      if (wave == 0) s_qi[r] = qix[t];
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(&s_acc[wave][r][16 * dt + 4 * g]) = acc[t][dt];
    __syncthreads();
    for (int pc = tid; pc < 16 * P4; pc += NT) {
      const int rr = pc / P4, c4 = pc - rr * P4;
      const int R = 16 * t + rr;
      if (R >= nrows) break;  // pieces go row by row: the rest are past the group too
      float M = s_m[0][rr];
#pragma unroll
      for (int w = 1; w < W; ++w) M = fmaxf(M, s_m[w][rr]);
      float ls = 0.f;
      f32x4 as = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float mw = s_m[w][rr];
        const float f = (mw == kNegInf) ? 0.f : fast_exp2((mw - M) * sl2);
        ls += s_l[w][rr] * f;
        as += *reinterpret_cast<const f32x4*>(&s_acc[w][rr][4 * c4]) * f;
      }
      const int j = R / G;
      const int h = kvh * G + (R - j * G);
      if (it.part_base < 0) {
        // divided, not multiplied by 1 / l: a single visible key then gives
        // its value exactly
        *reinterpret_cast<f32x4*>(a.out + (static_cast<size_t>(s_qi[rr]) * a.hq + h) * D + 4 * c4) = as / ls;
      } else if ((it.qmask >> j) & 1ull) {
        const size_t slot = static_cast<size_t>(it.part_base) + static_cast<size_t>(j) * a.hq + h;
        *reinterpret_cast<f32x4*>(a.part_acc + slot * D + 4 * c4) = as;
        if (c4 == 0) {
          a.part_ml[2 * slot] = M;
          a.part_ml[2 * slot + 1] = ls;
        }
      }
    }
    __syncthreads();
  }
}

template <class P, int D, int T, int W, bool C, class X>
void note_partial() {
  char nm[112];
  snprintf(nm, sizeof nm, "attn_partial_kernel<%s, %d, %d, %d, %s%s>", P::kName, D, T, W, C ? "true" : "false",
           X::kActive ? ", NewTokens" : "");
  launch_log_add(nm);
}

template <class P, int D, int T, int W, bool C, class X>
hipError_t launch_one(const AttnArgs& args, const X& x, int32_t n_items, hipStream_t s) {
  hipLaunchKernelGGL((attn_partial_kernel<P, D, T, W, C, X>), dim3(n_items * args.hkv), dim3(64 * W), 0, s, args, x);
  note_partial<P, D, T, W, C, X>();
  return hipGetLastError();
}

// Eight waves only at one tile and not for fp32 at d = 128 (more fragments per
// wave than eight waves leave registers for); two waves at one tile; four
// otherwise.
template <class P, int D, bool C, class X>
hipError_t launch_w(int tiles, int waves, const AttnArgs& args, const X& x, int32_t n_items, hipStream_t s) {
  if constexpr (kIsBF16<P> || D <= 64) {
    if (waves == 8 && tiles == 1) return launch_one<P, D, 1, 8, C, X>(args, x, n_items, s);
  }
  if (waves == 2 && tiles == 1) return launch_one<P, D, 1, 2, C, X>(args, x, n_items, s);
  if (tiles == 1) return launch_one<P, D, 1, 4, C, X>(args, x, n_items, s);
  if (tiles == 2) return launch_one<P, D, 2, 4, C, X>(args, x, n_items, s);
  return hipErrorInvalidValue;
}

template <class P, int D>
hipError_t launch_c(int tiles, int waves, bool causal, const AttnArgs& args, const NewTokens* nt, int32_t n_items,
                    hipStream_t s) {
  if (nt)
    return causal ? launch_w<P, D, true, NewTokens>(tiles, waves, args, *nt, n_items, s)
                  : launch_w<P, D, false, NewTokens>(tiles, waves, args, *nt, n_items, s);
  return causal ? launch_w<P, D, true, NoNewTokens>(tiles, waves, args, NoNewTokens{}, n_items, s)
                : launch_w<P, D, false, NoNewTokens>(tiles, waves, args, NoNewTokens{}, n_items, s);
}

}  // namespace

hipError_t launch_attn_partial(int dtype, int head_dim, int tiles, int waves, bool causal, const AttnArgs& args,
                               int32_t n_items, hipStream_t stream, const NewTokens* nt) {
  if (n_items <= 0) return hipSuccess;
  if (waves != 2 && waves != 4 && waves != 8) return hipErrorInvalidValue;
  if (dtype == 1 && head_dim == 128) return launch_c<BF16, 128>(tiles, waves, causal, args, nt, n_items, stream);
  if (dtype == 1 && head_dim == 64) return launch_c<BF16, 64>(tiles, waves, causal, args, nt, n_items, stream);
  if (dtype == 0 && head_dim == 128) return launch_c<F32, 128>(tiles, waves, causal, args, nt, n_items, stream);
  if (dtype == 0 && head_dim == 64) return launch_c<F32, 64>(tiles, waves, causal, args, nt, n_items, stream);
  return hipErrorInvalidValue;
}

}  // namespace tkv
