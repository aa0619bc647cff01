// Append-scatter and gather kernels for the pool tiles, and the in-place plan update.
//
// tkv_append writes each new token's K and V once into its block slot (DSpark
// blog, third layer: each token's KV is computed once and reused).  One
// workgroup builds one (block, KV head, layer) tile: it stages the new tokens'
// rows in LDS with 16-byte loads, then writes the tile's 16-byte chunks in the
// pool's element order (layout.h).  A block that this append opens is written
// whole, with zeros in the slots no token fills yet, so no slot ever holds
// uninitialised bits; a block that continues keeps its earlier slots.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "kernels.h"
#include "layout.h"

namespace tkv {
namespace {

template <int EB>
struct Elem;
template <>
struct Elem<2> {
  using T = uint16_t;
};
template <>
struct Elem<4> {
  using T = uint32_t;
};

// One entry's tokens in one (layer, KV head) tile: source rows [ent.src,
// ent.src + ent.cnt) of the [L][ntok][Hkv][D] arrays go to slots [ent.slot,
// ...) of block ent.blk; a fresh block (slot 0) is written whole.  Called by
// every thread of a 256-thread workgroup.
template <int EB, int D, class Args>
__device__ void write_tile(const Args& a, const AppendEntry ent, int kvh, int layer) {
  using L = Layout<EB>;
  using E = typename Elem<EB>::T;
  constexpr int PC = L::kPerChunk;
  constexpr int NCH = 16 * D / PC;
  constexpr int CPR = D / PC;  // chunks per token row
  __shared__ __align__(16) E sk[16 * D];
  __shared__ __align__(16) E sv[16 * D];

  const int tid = threadIdx.x;
  const int slot_lo = ent.slot, src0 = ent.src, cnt = ent.cnt;
  const bool fresh = slot_lo == 0;
  if (cnt <= 0 || slot_lo + cnt > 16) return;

  const E* srck = static_cast<const E*>(a.src_k);
  const E* srcv = static_cast<const E*>(a.src_v);
  for (int idx = tid; idx < cnt * CPR; idx += 256) {
    const int t = idx / CPR, c = idx - t * CPR;
    const size_t so = ((static_cast<size_t>(layer) * a.ntok + src0 + t) * a.hkv + kvh) * D + c * PC;
    const int lo = (slot_lo + t) * D + c * PC;
    *reinterpret_cast<uint4*>(&sk[lo]) = *reinterpret_cast<const uint4*>(srck + so);
    *reinterpret_cast<uint4*>(&sv[lo]) = *reinterpret_cast<const uint4*>(srcv + so);
  }
  __syncthreads();

  const size_t base = static_cast<size_t>(layer) * a.layer_stride +
                      (static_cast<size_t>(ent.blk) * a.hkv + kvh) * (16 * D);
  uint4* kt = reinterpret_cast<uint4*>(static_cast<E*>(a.kpool) + base);
  uint4* vt = reinterpret_cast<uint4*>(static_cast<E*>(a.vpool) + base);
  const int hi = slot_lo + cnt;
  for (int ch = tid; ch < NCH; ch += 256) {
    // K: a chunk holds one token
    {
      int tok, d;
      L::k_coord(ch, 0, tok, d);
      const bool isnew = tok >= slot_lo && tok < hi;
      if (isnew || fresh) {
        E vals[PC];
#pragma unroll
        for (int el = 0; el < PC; ++el) {
          L::k_coord(ch, el, tok, d);
          vals[el] = isnew ? sk[tok * D + d] : E(0);
        }
        kt[ch] = *reinterpret_cast<uint4*>(vals);
      }
    }
    // V: a chunk holds four consecutive tokens
    {
      bool anynew = false;
#pragma unroll
      for (int el = 0; el < PC; ++el) {
        int tok, d;
        L::v_coord(ch, el, tok, d);
        anynew |= tok >= slot_lo && tok < hi;
      }
      if (anynew || fresh) {
        E vals[PC];
        if (!fresh) *reinterpret_cast<uint4*>(vals) = vt[ch];
#pragma unroll
        for (int el = 0; el < PC; ++el) {
          int tok, d;
          L::v_coord(ch, el, tok, d);
          if (tok >= slot_lo && tok < hi) vals[el] = sv[tok * D + d];
          else if (fresh) vals[el] = E(0);
        }
        vt[ch] = *reinterpret_cast<uint4*>(vals);
      }
    }
  }
}

template <int EB, int D>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  write_tile<EB, D>(a, a.ent[blockIdx.x], blockIdx.y, blockIdx.z);
}

// The new tokens of a decode step in one layer (workgroups x < nent, one per
// entry and KV head), and the changed words of the call's plan (the
// workgroup after them, with y = 0): everything the step's attention launch
// needs written before it, in one launch.
template <int EB, int D>
__global__ __launch_bounds__(256) void decode_prep_kernel(DecodePrepArgs a) {
  if (static_cast<int32_t>(blockIdx.x) < a.app.nent) {
    write_tile<EB, D>(a.app, a.app.ent[blockIdx.x], blockIdx.y, 0);  // app's pools are the layer's
    return;
  }
  if (blockIdx.y != 0) return;
  for (int32_t i = static_cast<int32_t>(threadIdx.x); i < a.npatch; i += 256) {
    const PlanWord w = a.patch[i];
    if (w.word < a.limit) a.plan[w.word] = w.value;
  }
}

template <int EB, int D>
__global__ __launch_bounds__(256) void gather_kernel(GatherArgs a) {
  using L = Layout<EB>;
  using E = typename Elem<EB>::T;
  constexpr int PC = L::kPerChunk;
  constexpr int NCH = 16 * D / PC;
  constexpr int CPR = D / PC;
  __shared__ __align__(16) E sk[16 * D];
  __shared__ __align__(16) E sv[16 * D];
  const int e = blockIdx.x, kvh = blockIdx.y, tid = threadIdx.x;
  const size_t base = (static_cast<size_t>(a.blk[e]) * a.hkv + kvh) * (16 * D);
  const uint4* kt = reinterpret_cast<const uint4*>(static_cast<const E*>(a.kpool) + base);
  const uint4* vt = reinterpret_cast<const uint4*>(static_cast<const E*>(a.vpool) + base);
  for (int ch = tid; ch < NCH; ch += 256) {
    E kv[PC], vv[PC];
    *reinterpret_cast<uint4*>(kv) = kt[ch];
    *reinterpret_cast<uint4*>(vv) = vt[ch];
#pragma unroll
    for (int el = 0; el < PC; ++el) {
      int tok, d;
      L::k_coord(ch, el, tok, d);
      sk[tok * D + d] = kv[el];
      L::v_coord(ch, el, tok, d);
      sv[tok * D + d] = vv[el];
    }
  }
  __syncthreads();
  const int valid = a.valid[e], pos = a.pos[e];
  E* ko = static_cast<E*>(a.k_out);
  E* vo = static_cast<E*>(a.v_out);
  for (int idx = tid; idx < valid * CPR; idx += 256) {
    const int t = idx / CPR, c = idx - t * CPR;
    const size_t oo = (static_cast<size_t>(pos + t) * a.hkv + kvh) * D + c * PC;
    *reinterpret_cast<uint4*>(ko + oo) = *reinterpret_cast<const uint4*>(&sk[t * D + c * PC]);
    *reinterpret_cast<uint4*>(vo + oo) = *reinterpret_cast<const uint4*>(&sv[t * D + c * PC]);
  }
}

// Writes a list of changed 32-bit words into a device plan (the in-place
// update after appends that fitted in their tip blocks): one word per thread,
// words at or past `limit` skipped.
__global__ __launch_bounds__(256) void plan_patch_kernel(int32_t* __restrict__ plan,
                                                         const PlanWord* __restrict__ words, int32_t n,
                                                         uint32_t limit) {
  const int32_t i = static_cast<int32_t>(blockIdx.x) * 256 + static_cast<int32_t>(threadIdx.x);
  if (i >= n) return;
  const PlanWord w = words[i];
  if (w.word < limit) plan[w.word] = w.value;
}

// Copies a serialised plan from pinned host memory into its device buffer:
// 16 bytes per thread and step (the loads cross the host link, all of a
// thread's in flight at once), then the last n4 4-byte words.
__global__ __launch_bounds__(256) void plan_copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                        int64_t n16, int32_t n4) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
  if (blockIdx.x == 0 && static_cast<int32_t>(threadIdx.x) < n4)
    reinterpret_cast<int32_t*>(dst + n16)[threadIdx.x] = reinterpret_cast<const int32_t*>(src + n16)[threadIdx.x];
}

// The same with the words in the kernel arguments.
__global__ __launch_bounds__(512) void plan_patch_args_kernel(PatchArgs a) {
  const int32_t i = static_cast<int32_t>(threadIdx.x);
  if (i >= a.n) return;
  const PlanWord w = a.w[i];
  if (w.word < a.limit) a.plan[w.word] = w.value;
}

}  // namespace

hipError_t launch_plan_patch_args(const PatchArgs& args, hipStream_t stream) {
  if (args.n <= 0 || args.n > kPatchArgWords) return hipErrorInvalidValue;
  hipLaunchKernelGGL(plan_patch_args_kernel, dim3(1), dim3(512), 0, stream, args);
  launch_log_add("plan_patch_args_kernel");
  return hipGetLastError();
}

hipError_t launch_plan_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return hipSuccess;
  if (bytes % 4 || (reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) % 16) return hipErrorInvalidValue;
  const int64_t n16 = static_cast<int64_t>(bytes / 16);
  const int32_t n4 = static_cast<int32_t>((bytes % 16) / 4);
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n16 + 255) / 256, 1024));
  hipLaunchKernelGGL(plan_copy_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                     static_cast<uint4*>(dst), static_cast<const uint4*>(src), n16, n4);
  launch_log_add("plan_copy_kernel");
  return hipGetLastError();
}

hipError_t launch_plan_patch(int32_t* plan, const PlanWord* words, int32_t n, uint32_t limit, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(plan_patch_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, plan, words, n, limit);
  launch_log_add("plan_patch_kernel");
  return hipGetLastError();
}

hipError_t launch_append(int dtype, int head_dim, int32_t layers, const AppendArgs& args,
                         hipStream_t stream) {
  const dim3 grid(args.nent, args.hkv, layers);
  if (dtype == 1 && head_dim == 128) hipLaunchKernelGGL((append_kernel<2, 128>), grid, dim3(256), 0, stream, args);
  else if (dtype == 1 && head_dim == 64) hipLaunchKernelGGL((append_kernel<2, 64>), grid, dim3(256), 0, stream, args);
  else if (dtype == 0 && head_dim == 128) hipLaunchKernelGGL((append_kernel<4, 128>), grid, dim3(256), 0, stream, args);
  else if (dtype == 0 && head_dim == 64) hipLaunchKernelGGL((append_kernel<4, 64>), grid, dim3(256), 0, stream, args);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode_prep(int dtype, int head_dim, const DecodePrepArgs& args, hipStream_t stream) {
  if (args.app.nent < 0 || args.app.nent > kAppendMaxBlocks || args.npatch < 0 || args.npatch > kPrepPatchWords)
    return hipErrorInvalidValue;
  const int extra = args.npatch > 0 ? 1 : 0;
  if (args.app.nent + extra == 0) return hipSuccess;
  const dim3 grid(args.app.nent + extra, args.app.hkv, 1);
  if (dtype == 1 && head_dim == 128) hipLaunchKernelGGL((decode_prep_kernel<2, 128>), grid, dim3(256), 0, stream, args);
  else if (dtype == 1 && head_dim == 64) hipLaunchKernelGGL((decode_prep_kernel<2, 64>), grid, dim3(256), 0, stream, args);
  else if (dtype == 0 && head_dim == 128) hipLaunchKernelGGL((decode_prep_kernel<4, 128>), grid, dim3(256), 0, stream, args);
  else if (dtype == 0 && head_dim == 64) hipLaunchKernelGGL((decode_prep_kernel<4, 64>), grid, dim3(256), 0, stream, args);
  else return hipErrorInvalidValue;
  launch_log_add("decode_prep_kernel");
  return hipGetLastError();
}

hipError_t launch_gather(int dtype, int head_dim, const GatherArgs& args, hipStream_t stream) {
  const dim3 grid(args.nent, args.hkv, 1);
  if (dtype == 1 && head_dim == 128) hipLaunchKernelGGL((gather_kernel<2, 128>), grid, dim3(256), 0, stream, args);
  else if (dtype == 1 && head_dim == 64) hipLaunchKernelGGL((gather_kernel<2, 64>), grid, dim3(256), 0, stream, args);
  else if (dtype == 0 && head_dim == 128) hipLaunchKernelGGL((gather_kernel<4, 128>), grid, dim3(256), 0, stream, args);
  else if (dtype == 0 && head_dim == 64) hipLaunchKernelGGL((gather_kernel<4, 64>), grid, dim3(256), 0, stream, args);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace tkv
