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
//     super-block keeps NS - 2 super-blocks in flight per wave;
//   * each wave reads the staged K and V fragments from LDS (conflict-free 16-B
//     lane-contiguous reads in the pool's MFMA operand order) and runs the same
//     S^T = K Q^T, online softmax and O^T += V^T P^T steps as attn.hip for each of
//     its tiles; a super-block no row of a wave can see is skipped by that wave;
//   * waves own disjoint rows, so no cross-wave merge is needed at the end.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_common.h"
#include "kernels.h"

namespace tkv {
namespace {

using namespace attn;

__device__ inline uint32_t lds_byte_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// One wave-load: lane i copies 16 bytes from src (its own address) to LDS byte
// address dst + 16 i.  dst must be wave-uniform.
__device__ inline void dma16(const void* src, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(dst) : "memory", "m0");
}

template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt vmcnt(n) for a wave-uniform n (an immediate must be spelled out).
template <int N = 0>
__device__ inline void wait_vm_dyn(int n) {
  if constexpr (N < 48) {
    if (n <= N) {
      wait_vm<N>();
      return;
    }
    wait_vm_dyn<N + 1>(n);
  } else {
    wait_vm<0>();
  }
}

// Workgroups per CU a shape is built for: two at one tile per wave, else one.
// Two workgroups hide each other's latency; one workgroup gets the deeper ring.
template <int TPW, int W>
constexpr int rows_wgs_per_cu() {
  return TPW == 1 ? 2 : 1;
}
// Waves per SIMD the register budget must allow.  The dispatcher places each
// workgroup's waves starting from the first SIMD, so two 6-wave workgroups can
// put 4 waves on one SIMD: shapes with more than 4 waves need 128 VGPRs.
template <int TPW, int W>
constexpr int rows_min_waves() {
  return rows_wgs_per_cu<TPW, W>() == 1 ? 1 : (W > 4 ? 4 : 2);
}

template <class P, int D, int TPW, int W, int NS, bool CAUSAL>
__global__ __launch_bounds__(64 * W, (rows_min_waves<TPW, W>())) void attn_rows_kernel(AttnArgs a) {
  using E = typename P::elem;
  using F = typename P::template Frag<D>;
  constexpr int NDT = D / 16;
  constexpr int TILE_BYTES = 16 * D * static_cast<int>(sizeof(E));
  constexpr int LPT = TILE_BYTES / 1024;  // wave-loads per tile
  constexpr int SB_LOADS = 4 * LPT;       // K a, K b, V a, V b
  constexpr int LPW_MAX = (SB_LOADS + W - 1) / W;  // wave-loads per wave per super-block
  constexpr int STAGE = SB_LOADS * 1024;
  __shared__ __attribute__((aligned(1024))) char ring[NS * STAGE];
  __shared__ DevBlock ents[kRowsMaxItemBlocks];  // the item's block list

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int kvh = blockIdx.x % a.hkv;
  const DevItem it = a.items[a.item0 + blockIdx.x / a.hkv];
  const int nb = it.blk_count;
  const int nsb = (nb + 1) >> 1;
  const DevBlock* bl = a.blocks + it.blk_begin;
  const size_t tile_elems = 16 * D;
  const size_t bstride = static_cast<size_t>(a.hkv) * tile_elems;
  const char* kbase = reinterpret_cast<const char*>(static_cast<const E*>(a.kpool) + kvh * tile_elems);
  const char* vbase = reinterpret_cast<const char*>(static_cast<const E*>(a.vpool) + kvh * tile_elems);
  const uint32_t ring_base = __builtin_amdgcn_readfirstlane(lds_byte_addr(ring));

  // the item's block list, staged once: the loader and every wave read block ids,
  // valid counts, positions and masks from here without touching global memory
  for (int k = tid; k < nb; k += 64 * W) ents[k] = bl[k];
  __syncthreads();

  // Issue this wave's share of super-block s's loads into ring slot `slot`.
  auto issue = [&](int s, int slot) {
    const int ida = __builtin_amdgcn_readfirstlane(ents[2 * s].id);
    const int idb = (2 * s + 1 < nb) ? __builtin_amdgcn_readfirstlane(ents[2 * s + 1].id) : ida;
#pragma unroll
    for (int k = 0; k < LPW_MAX; ++k) {
      const int i = wave + W * k;
      if (i >= SB_LOADS) break;
      const int t = i / LPT, part = i - t * LPT;
      const int id = (t & 1) ? idb : ida;
      const char* base = (t & 2) ? vbase : kbase;
      const char* src = base + (static_cast<size_t>(id) * bstride) * sizeof(E) + part * 1024 + lane * 16;
      dma16(src, ring_base + slot * STAGE + i * 1024);
    }
  };

  // rows of this wave: tiles wave, wave + W, ...
  const DevGroup gr = a.groups[it.group];
  const int G = a.gsize;
  const int nrows = gr.nq * G;
  const uint64_t gmask = gr.nq >= 64 ? ~0ull : ((1ull << gr.nq) - 1);
  F qf[TPW];
  int qj[TPW], qlim[TPW];
  uint64_t my_q = 0;  // group queries with a row in this wave's tiles
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tile = wave + W * t;
    const int R = 16 * tile + r;
    if (16 * tile < nrows) {
      const int j0 = (16 * tile) / G, j1 = min(nrows - 1, 16 * tile + 15) / G;
      for (int j = j0; j <= j1; ++j) my_q |= 1ull << j;
    }
    if (R < nrows) {
      const int j = R / G;
      const int h = kvh * G + (R - j * G);
      const int qi = a.gq[gr.q_begin + j];
      P::load_q(qf[t], static_cast<const E*>(a.q) + (static_cast<size_t>(qi) * a.hq + h) * D, g);
      qj[t] = j;
      qlim[t] = CAUSAL ? a.gqpos[gr.q_begin + j] : 0;
    } else {
      P::zero(qf[t]);
      qj[t] = 0;
      qlim[t] = 0x7fffffff;
    }
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
  const int min_lim = gr.min_pos;
  const bool active = 16 * wave < nrows;

  // Every load the compiler can see (queries, group data, the block list) is
  // complete here, and it knows it, so it places no vmcnt waits of its own in
  // the loop below: those would also count our invisible ring loads and drain
  // the ring on every iteration.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (nsb > 0) {
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(min(s, nsb - 1), s);
  }

  // this wave's share of a super-block's loads (waves below SB_LOADS % W take one more)
  const int my_loads = (SB_LOADS - wave + W - 1) / W;
  const int ring_wait = (NS - 2) * my_loads;
  for (int s = 0; s < nsb; ++s) {
    if constexpr (SB_LOADS % W == 0) wait_vm<(NS - 2) * (SB_LOADS / W)>();
    else wait_vm_dyn(ring_wait);
    __builtin_amdgcn_s_barrier();
    issue(min(s + NS - 1, nsb - 1), (s + NS - 1) % NS);

    // metadata of super-block s
    const int ba = 2 * s, bbk = 2 * s + 1;
    SBMeta e;
    e.va = __builtin_amdgcn_readfirstlane(ents[ba].valid);
    e.pa = __builtin_amdgcn_readfirstlane(ents[ba].pos);
    {
      const uint64_t mk = ents[ba].mask;
      e.ma = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(mk >> 32))) << 32) |
             static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(mk)));
    }
    if (bbk < nb) {
      e.vb = __builtin_amdgcn_readfirstlane(ents[bbk].valid);
      e.pb = __builtin_amdgcn_readfirstlane(ents[bbk].pos);
      const uint64_t mk = ents[bbk].mask;
      e.mb = (static_cast<uint64_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(mk >> 32))) << 32) |
             static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(mk)));
    } else {
      e.vb = 0;
      e.pb = e.pa;
      e.mb = 0;
    }
    if (!active || ((e.ma | e.mb) & my_q) == 0) continue;

    const char* st = ring + (s % NS) * STAGE;
    F ka, kb, va, vb;
    P::load_tile_lds(ka, st + 0 * TILE_BYTES, lane);
    P::load_tile_lds(kb, st + 1 * TILE_BYTES, lane);
    [[maybe_unused]] u32x4 av[NDT];
    const bool see_a = (e.ma & gmask) == gmask, see_b = (e.mb & gmask) == gmask;
    const bool need_mask = e.va < 16 || e.vb < 16 || !see_a || !see_b ||
                           (CAUSAL && (e.pa + 15 > min_lim || e.pb + 15 > min_lim));
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      if (16 * (wave + W * t) >= nrows) break;
      const f32x4 sa = P::qk(ka, qf[t]);
      const f32x4 sb = P::qk(kb, qf[t]);
      if (t == 0) {
        // V fragments are read only once the K fragments are consumed, so the two
        // are never live together (one tile per wave then fits 128 VGPRs)
        if constexpr (TPW == 1) __builtin_amdgcn_sched_barrier(0);
        if constexpr (kIsBF16<P>) {
          P::template lds_av<D>(av, st + 2 * TILE_BYTES, st + 3 * TILE_BYTES, lane);
        } else {
          P::load_tile_lds(va, st + 2 * TILE_BYTES, lane);
          P::load_tile_lds(vb, st + 3 * TILE_BYTES, lane);
        }
      }
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
      float bm = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
      bm = fmaxf(bm, __shfl_xor(bm, 16));
      bm = fmaxf(bm, __shfl_xor(bm, 32));
      // m is kept in raw score units; exponents are (s - m) * log2(e) / sqrt(D)
      const float mn = fmaxf(m[t], bm);
      if (__any(mn > m[t] + tau_raw)) {
        const float alpha = (m[t] == kNegInf) ? 0.f : fast_exp2((m[t] - mn) * sl2);
        l[t] *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) acc[t][dt] *= alpha;
        m[t] = mn;
      }
      const float mc = (m[t] == kNegInf) ? 0.f : m[t] * sl2;
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = fast_exp2(fmaf(sc[i], sl2, -mc));
      if constexpr (kIsBF16<P>) P::template pv2_av<D>(av, p, acc[t], l[t]);
      else P::pv2(va, vb, p, acc[t], l[t]);
    }
  }
  // every DMA this wave issued must land before the workgroup's LDS is released
  wait_vm<0>();
  mfma_result_fence();

  // write this wave's rows: lane (g, r) holds O^T[16 dt + 4 g + i][row r]
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int tile = wave + W * t;
    if (16 * tile >= nrows) break;
    float lt = l[t];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int R = 16 * tile + r;
    if (R >= nrows) continue;
    const int j = R / G;
    const int h = kvh * G + (R - j * G);
    if (it.part_base < 0) {
      const int qi = a.gq[gr.q_begin + j];
      float* o = a.out + (static_cast<size_t>(qi) * a.hq + h) * D;
      const float inv = 1.f / lt;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4*>(o + 16 * dt + 4 * g) = acc[t][dt] * inv;
    } else {
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

// Ring depth: as many super-blocks as fit in 64 KiB (two workgroups per CU) or
// 128 KiB (one), at most 8; with the 12 KiB block list either fits the CU's
// 160 KiB of LDS.
template <class P, int D, int WGS>
constexpr int ring_stages() {
  constexpr int stage = 4 * 16 * D * static_cast<int>(sizeof(typename P::elem));
  constexpr int budget = (WGS == 2 ? 64 : 128) * 1024;
  return (budget / stage) < 8 ? (budget / stage) : 8;
}

template <class P, int D, int TPW, int W, bool C>
hipError_t launch_one(const AttnArgs& args, int32_t n_items, hipStream_t s) {
  constexpr int NS = ring_stages<P, D, rows_wgs_per_cu<TPW, W>()>();
  hipLaunchKernelGGL((attn_rows_kernel<P, D, TPW, W, NS, C>), dim3(n_items * args.hkv), dim3(64 * W), 0, s, args);
  return hipGetLastError();
}

template <class P, int D, bool C>
hipError_t launch_shape(int tiles, const AttnArgs& args, int32_t n_items, hipStream_t s) {
  if (tiles <= 4) return launch_one<P, D, 1, 4, C>(args, n_items, s);
  if (tiles <= 6) return launch_one<P, D, 1, 6, C>(args, n_items, s);
  if (tiles <= 8) return launch_one<P, D, 1, 8, C>(args, n_items, s);
  if (tiles <= 16) return launch_one<P, D, 2, 8, C>(args, n_items, s);
  return hipErrorInvalidValue;
}

template <class P, int D>
hipError_t launch_c(int tiles, bool causal, const AttnArgs& args, int32_t n_items, hipStream_t s) {
  return causal ? launch_shape<P, D, true>(tiles, args, n_items, s) : launch_shape<P, D, false>(tiles, args, n_items, s);
}

}  // namespace

hipError_t launch_attn_rows(int dtype, int head_dim, int tiles, bool causal, const AttnArgs& args, int32_t n_items,
                            hipStream_t stream) {
  if (n_items <= 0) return hipSuccess;
  if (dtype == 1 && head_dim == 128) return launch_c<BF16, 128>(tiles, causal, args, n_items, stream);
  if (dtype == 1 && head_dim == 64) return launch_c<BF16, 64>(tiles, causal, args, n_items, stream);
  if (dtype == 0 && head_dim == 128) return launch_c<F32, 128>(tiles, causal, args, n_items, stream);
  if (dtype == 0 && head_dim == 64) return launch_c<F32, 64>(tiles, causal, args, n_items, stream);
  return hipErrorInvalidValue;
}

}  // namespace tkv
