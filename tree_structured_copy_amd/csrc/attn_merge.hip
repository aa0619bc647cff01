// Log-sum-exp merge of split-K and cascade partials (flash-decoding style).
//
// A query whose path was cut into several work items -- chunks of a long
// block list, or the shared and the private part of a search tree's path --
// has one partial record per item: the running maximum m (raw score units),
// the sum l of exp2((s - m) * log2(e)/sqrt(d)) and the unnormalised sum acc of
// those weights times V.  This pass combines them into the normalised output.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_common.h"
#include "kernels.h"

namespace tkv {
namespace {

using namespace attn;

// Log-sum-exp merge: one wave per (query, query head).  Lane c takes partial
// c's record (slot, m, l), the wave forms the common maximum M, and then every
// lane accumulates its D/64 output elements over the partials, each weighted
// by exp2((m_c - M) * scale_log2); the sum of the weighted l_c normalises.
// The first 64 records' fields stay in registers between the two passes (most
// queries have fewer), and the acc rows are loaded kBatch at a time before any
// is used, so a wave waits for one round trip per batch, not per record.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs a) {
  constexpr int PER = D / 64;  // output elements per lane
  constexpr int kBatch = 8;
  using VT = typename std::conditional<PER == 2, float2, float>::type;
  const int lane = threadIdx.x & 63;
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= a.nq * a.hq) return;
  const int q = w / a.hq, h = w - q * a.hq;
  const DevMerge mg = a.merge[q];
  if (mg.p_count == 0) return;
  const float sl2 = a.scale_log2;
  int slot_r = 0;
  float m_r = kNegInf, l_r = 0.f;
  if (lane < mg.p_count) {
    slot_r = a.parts[mg.p_begin + lane].slot0 + h;
    m_r = a.part_ml[2 * slot_r];
    l_r = a.part_ml[2 * slot_r + 1];
  }
  float M = m_r;
  for (int c0 = 64; c0 < mg.p_count; c0 += 64) {
    const int c = c0 + lane;
    if (c < mg.p_count) M = fmaxf(M, a.part_ml[2 * (a.parts[mg.p_begin + c].slot0 + h)]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float ls = 0.f;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int c0 = 0; c0 < mg.p_count; c0 += 64) {
    const int c = c0 + lane;
    int slot = slot_r;
    float mc = m_r, lc = l_r;
    if (c0 > 0) {
      slot = 0;
      mc = kNegInf;
      lc = 0.f;
      if (c < mg.p_count) {
        slot = a.parts[mg.p_begin + c].slot0 + h;
        mc = a.part_ml[2 * slot];
        lc = a.part_ml[2 * slot + 1];
      }
    }
    const float f = (mc == kNegInf) ? 0.f : fast_exp2((mc - M) * sl2);
    ls += lc * f;
    const int cnt = min(64, mg.p_count - c0);
    for (int k0 = 0; k0 < cnt; k0 += kBatch) {
      VT v[kBatch];
      float fk[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        // past the end: the last record again, with weight 0 (no branch, so
        // the batch's loads all issue before the first wait)
        const int k = min(k0 + u, cnt - 1);
        const int sk = __builtin_amdgcn_readlane(slot, k);
        const float fu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), k));
        fk[u] = (k0 + u < cnt) ? fu : 0.f;
        v[u] = *reinterpret_cast<const VT*>(a.part_acc + static_cast<size_t>(sk) * D + lane * PER);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if constexpr (PER == 2) {
          acc[0] += v[u].x * fk[u];
          acc[1] += v[u].y * fk[u];
        } else {
          acc[0] += v[u] * fk[u];
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o);
  const float inv = 1.f / ls;
  float* dst = a.out + (static_cast<size_t>(q) * a.hq + h) * D + lane * PER;
  if constexpr (PER == 2) {
    *reinterpret_cast<float2*>(dst) = make_float2(acc[0] * inv, acc[1] * inv);
  } else {
    dst[0] = acc[0] * inv;
  }
}

}  // namespace

hipError_t launch_attn_merge(int head_dim, const MergeArgs& args, hipStream_t stream) {
  if (args.nq <= 0) return hipSuccess;
  const dim3 grid((args.nq * args.hq + 3) / 4);  // four waves, four (query, head) pairs per workgroup
  if (head_dim == 128) hipLaunchKernelGGL((attn_merge_kernel<128>), grid, dim3(256), 0, stream, args);
  else if (head_dim == 64) hipLaunchKernelGGL((attn_merge_kernel<64>), grid, dim3(256), 0, stream, args);
  else return hipErrorInvalidValue;
  launch_log_add(head_dim == 128 ? "attn_merge_kernel<128>" : "attn_merge_kernel<64>");
  return hipGetLastError();
}

}  // namespace tkv
