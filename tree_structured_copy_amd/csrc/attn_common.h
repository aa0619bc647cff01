// Shared pieces of the attention kernels: MFMA operand policies per input
// dtype and small device helpers.  Included by attn.hip and attn_rows.hip only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tkv_types.h"

namespace tkv {
namespace attn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kTau = 8.0f;

template <class To, class From>
__device__ inline To bitcast(const From& f) {
  return __builtin_bit_cast(To, f);
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS reads by byte address (the address of a __shared__ object plus an offset).
template <class T>
__device__ inline T lds_ld(uint32_t addr) {
  return *(const __attribute__((address_space(3))) T*)(addr);
}
// The same read kept apart from its neighbours: the compiler neither merges it
// with an adjacent read nor reorders it across another volatile LDS read.
template <class T>
__device__ inline T lds_ld_sep(uint32_t addr) {
  return *(const volatile __attribute__((address_space(3))) T*)(addr);
}

// Split 8 fp32 weights into bf16 hi = bf16(p) (round to nearest even) and
// lo = bf16(p - hi): hi + lo carries p to about 2^-17 relative.  Packed
// conversions, and the fp32 value of each hi recovered by a shift or a mask.
__device__ inline void split_hi_lo(const float* p, bf16x8& hi, bf16x8& lo) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  u32x4 h, w;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x2 pj = {p[2 * j], p[2 * j + 1]};
    const uint32_t hj = bitcast<uint32_t>(__builtin_convertvector(pj, bf16x2));
    const f32x2 rem = {pj.x - bitcast<float>(hj << 16), pj.y - bitcast<float>(hj & 0xffff0000u)};
    h[j] = hj;
    w[j] = bitcast<uint32_t>(__builtin_convertvector(rem, bf16x2));
  }
  hi = bitcast<bf16x8>(h);
  lo = bitcast<bf16x8>(w);
}

// Wait states between an MFMA chain and the first VALU / accvgpr read of its
// result.  For v_mfma_f32_16x16x4_f32 on gfx950 the compiler's hazard model
// leaves too few (the last accumulator register was read before the final MFMA
// had written it: measured as missing terms in one score element), so the
// distance is enforced here: 24 wait states, more than the 19 that the longest
// (16-pass) XDL result needs, with scheduling barriers so nothing moves across.
__device__ inline void mfma_result_fence() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// bf16 inputs: S^T and O^T via 16x16x32 bf16 MFMAs.
struct BF16 {
  using elem = uint16_t;
  template <int D>
  struct Frag {
    u32x4 v[D / 32];
  };
  template <int D>
  __device__ static void load_tile(Frag<D>& f, const elem* tile, int lane) {
    const u32x4* p = reinterpret_cast<const u32x4*>(tile) + lane;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) f.v[i] = __builtin_nontemporal_load(p + i * 64);
  }
  template <int D>
  __device__ static void load_tile_lds(Frag<D>& f, uint32_t tile_addr, int lane) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) f.v[i] = lds_ld<u32x4>(tile_addr + (i * 64 + lane) * 16);
  }
  template <int D>
  __device__ static void load_q(Frag<D>& f, const elem* row, int g) {
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) f.v[kk] = *reinterpret_cast<const u32x4*>(row + 32 * kk + 8 * g);
  }
  template <int D>
  __device__ static void zero(Frag<D>& f) {
#pragma unroll
    for (int i = 0; i < D / 32; ++i) f.v[i] = u32x4{0u, 0u, 0u, 0u};
  }
  template <int D>
  __device__ static f32x4 qk(const Frag<D>& k, const Frag<D>& q) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(k.v[kk]), bitcast<bf16x8>(q.v[kk]), s, 0, 0, 0);
    return s;
  }
  // acc[dt] += V^T[16dt..16dt+15][4 tokens] . P^T.  A weight p is split into
  // bf16 hi = bf16(p) and lo = bf16(p - hi), so hi + lo carries p to about
  // 2^-17 relative; one 16x16x32 MFMA per d-tile takes k = (4 tokens, hi) and
  // (the same 4 tokens, lo), with the lane's V^T fragment given twice.
  template <int D>
  __device__ static void pv(const Frag<D>& v, const float* p, f32x4* acc, float& l) {
    l += (p[0] + p[1]) + (p[2] + p[3]);
    bf16x8 pb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 hi = static_cast<__bf16>(p[i]);
      pb[i] = hi;
      pb[4 + i] = static_cast<__bf16>(p[i] - static_cast<float>(hi));
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const u32x4 w = v.v[dt >> 1];
      const u32x4 a = (dt & 1) ? u32x4{w.z, w.w, w.z, w.w} : u32x4{w.x, w.y, w.x, w.y};
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(a), pb, acc[dt], 0, 0, 0);
    }
  }
  // Two blocks at once: k = 4 tokens of block a and 4 of block b; one MFMA
  // per d-tile for the hi parts of the weights and one for the lo parts.  The
  // P.V A operands are given ready-made (av[dt] = V^T fragments of a and b).
  template <int D>
  __device__ static void pv2_av(const u32x4* av, const float* p, f32x4* acc, float& l) {
    l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    bf16x8 hi, lo;
    split_hi_lo(p, hi, lo);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(av[dt]), hi, acc[dt], 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(av[dt]), lo, acc[dt], 0, 0, 0);
  }
  // The A operands of pv2_av for d-tile dt, read straight from two staged V
  // tiles in LDS: 8 bytes of block a and 8 bytes of block b per lane.
  template <int D>
  // The V tile of block b follows that of block a in LDS.
  __device__ static void lds_av(u32x4* av, uint32_t va_addr, int lane) {
    constexpr uint32_t kTileBytes = 16 * D * 2;
    uint32_t base = va_addr + lane * 16;
    asm volatile("" : "+v"(base));  // one address register; the rest are offsets
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const uint32_t off = (dt >> 1) * 1024 + (dt & 1) * 8;
      // two separate 8-byte reads that land in the halves of av[dt]; merged into
      // one 16-byte read (adjacent d-tiles) they would cost register moves
      const u32x2 x = lds_ld_sep<u32x2>(base + off);
      const u32x2 y = lds_ld_sep<u32x2>(base + kTileBytes + off);
      av[dt] = u32x4{x.x, x.y, y.x, y.y};
    }
  }
  template <int D>
  __device__ static void pv2(const Frag<D>& va, const Frag<D>& vb, const float* p, f32x4* acc, float& l) {
    l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    bf16x8 hi, lo;
    split_hi_lo(p, hi, lo);
    u32x4 av[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const u32x4 wa = va.v[dt >> 1], wb = vb.v[dt >> 1];
      av[dt] = (dt & 1) ? u32x4{wa.z, wa.w, wb.z, wb.w} : u32x4{wa.x, wa.y, wb.x, wb.y};
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(av[dt]), hi, acc[dt], 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(av[dt]), lo, acc[dt], 0, 0, 0);
  }
};

// fp32 inputs: 16x16x4 fp32 MFMAs (full fp32 products and sums).
struct F32 {
  using elem = float;
  template <int D>
  struct Frag {
    f32x4 v[D / 16];
  };
  template <int D>
  __device__ static void load_tile(Frag<D>& f, const elem* tile, int lane) {
    const f32x4* p = reinterpret_cast<const f32x4*>(tile) + lane;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) f.v[i] = __builtin_nontemporal_load(p + i * 64);
  }
  template <int D>
  __device__ static void load_tile_lds(Frag<D>& f, uint32_t tile_addr, int lane) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) f.v[i] = lds_ld<f32x4>(tile_addr + (i * 64 + lane) * 16);
  }
  template <int D>
  __device__ static void load_q(Frag<D>& f, const elem* row, int g) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) f.v[c] = *reinterpret_cast<const f32x4*>(row + 16 * c + 4 * g);
  }
  template <int D>
  __device__ static void zero(Frag<D>& f) {
#pragma unroll
    for (int i = 0; i < D / 16; ++i) f.v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  template <int D>
  __device__ static f32x4 qk(const Frag<D>& k, const Frag<D>& q) {
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < D / 16; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) s = __builtin_amdgcn_mfma_f32_16x16x4f32(k.v[c][j], q.v[c][j], s, 0, 0, 0);
    mfma_result_fence();
    return s;
  }
  template <int D>
  __device__ static void pv(const Frag<D>& v, const float* p, f32x4* acc, float& l) {
    l += (p[0] + p[1]) + (p[2] + p[3]);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v.v[dt][i], p[i], acc[dt], 0, 0, 0);
  }
  template <int D>
  __device__ static void pv2(const Frag<D>& va, const Frag<D>& vb, const float* p, f32x4* acc, float& l) {
    pv(va, p, acc, l);
    pv(vb, p + 4, acc, l);
  }
};

// Metadata of one super-block (two consecutive blocks of the item's list),
// wave-uniform.  idb == ida and vb == 0 when the list has an odd tail.
struct SBMeta {
  int ida, idb;
  int va, vb;
  int pa, pb;
  uint64_t ma, mb;
};

template <class P>
constexpr bool kIsBF16 = sizeof(typename P::elem) == 2;

}  // namespace attn
}  // namespace tkv
