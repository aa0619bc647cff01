// Shared pieces of the attention kernels: MFMA operand policies per input
// dtype and small device helpers.  Included by attn.hip and attn_rows.hip only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"
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
// The hi part alone: bf16(p) for 8 fp32 weights, round to nearest even.
__device__ inline void to_bf16(const float* p, bf16x8& hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  u32x4 h;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x2 pj = {p[2 * j], p[2 * j + 1]};
    h[j] = bitcast<uint32_t>(__builtin_convertvector(pj, bf16x2));
  }
  hi = bitcast<bf16x8>(h);
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

// ---- direct-to-LDS loads (global_load_lds_dwordx4) -------------------------
//
// The loads are issued from inline asm so that the waits are ours: the compiler
// would otherwise wait for every outstanding LDS DMA at each barrier.  The
// kernels that use them keep every compiler-visible global load out of their
// loops, so vmcnt counts only these loads there.

__device__ inline uint32_t lds_byte_addr(const void* p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// One wave-load: lane i copies the 16 bytes at sbase + voff (voff its own) to
// LDS byte address dst + 16 i.  sbase and dst must be wave-uniform.  The data
// is read once, so the load is marked nontemporal (streamed past the caches
// rather than kept in them): measured 5.3 -> 6.1 TB/s for the ring alone.
__device__ inline void dma16(const void* sbase, uint32_t voff, uint32_t dst) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(dst)
               : "memory", "m0");
}

template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ inline const char* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const char*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Wave-loads per loading wave: the smallest divisor of a super-block's loads
// that W waves can cover.  Waves [0, loads / LPW) load LPW each and the rest
// none, so every loading wave waits for the same count.
template <int LOADS, int W>
constexpr int rows_loads_per_wave() {
  int d = 1;
  while (d * W < LOADS || LOADS % d != 0) ++d;
  return d;
}

// bf16 inputs: S^T and O^T via 16x16x32 bf16 MFMAs.
struct BF16 {
  using elem = uint16_t;
  static constexpr const char* kName = "BF16";
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
  // The V side of one super-block: vp.av[dt] is the A operand of the P.V MFMA
  // for d-tile dt, V^T[16 dt + dl][4 tokens of block a, 4 tokens of block b]
  // for lane (g, dl): one 8-byte unit of each block's V tile (the pool keeps
  // unit dt*64 + lane of a tile at byte 8 (dt*64 + lane), layout.h), so both
  // halves load straight into place and every wave load is one contiguous
  // 512-byte run.
  template <int D>
  struct VPair {
    u32x4 av[D / 16];
  };
  template <int D>
  __device__ static void load_vpair(VPair<D>& v, const elem* va_tile, const elem* vb_tile, int lane) {
    const u32x2* pa = reinterpret_cast<const u32x2*>(va_tile) + lane;
    const u32x2* pb = reinterpret_cast<const u32x2*>(vb_tile) + lane;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const u32x2 x = __builtin_nontemporal_load(pa + dt * 64);
      const u32x2 y = __builtin_nontemporal_load(pb + dt * 64);
      v.av[dt] = u32x4{x.x, x.y, y.x, y.y};
    }
  }
  // The same from two staged V tiles in LDS (block b's right after block a's).
  template <int D>
  __device__ static void lds_vpair(VPair<D>& v, uint32_t va_addr, int lane) {
    constexpr uint32_t kTileBytes = 16 * D * 2;
    uint32_t base = va_addr + lane * 8;
    asm volatile("" : "+v"(base));  // one address register; the rest are offsets
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      // separate reads (never merged with a neighbour) into the halves of av[dt]
      const u32x2 x = lds_ld_sep<u32x2>(base + dt * 512);
      const u32x2 y = lds_ld_sep<u32x2>(base + kTileBytes + dt * 512);
      v.av[dt] = u32x4{x.x, x.y, y.x, y.y};
    }
  }
  // acc[dt] += V^T . P^T over the super-block's 8 tokens per lane group.  Each
  // weight p enters one MFMA per d-tile as bf16 hi = bf16(p) (relative error at
  // most 2^-9).  While some lane of the wave holds a weight above kLoShare of
  // its running sum l (the first super-blocks of a row, short contexts, weights
  // gathered on a few keys), the remainder lo = bf16(p - hi) goes through a
  // second MFMA per d-tile with the same A operand, carrying p to about 2^-17.
  // Once every weight is a small share of its sum, the rounding errors of many
  // comparable weights average out and hi alone stays far inside the output
  // tolerance.  pmax is the largest of the lane's 8 weights.
  static constexpr float kLoShare = 0.125f;
  template <int D>
  __device__ static void pv(const VPair<D>& v, const float* p, float pmax, f32x4* acc, float& l) {
    l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    bf16x8 hi, lo;
    const bool with_lo = __any(pmax > kLoShare * l);
    if (with_lo) split_hi_lo(p, hi, lo);
    else to_bf16(p, hi);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(v.av[dt]), hi, acc[dt], 0, 0, 0);
    if (with_lo) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(v.av[dt]), lo, acc[dt], 0, 0, 0);
    }
  }
};

// fp32 inputs: 16x16x4 fp32 MFMAs (full fp32 products and sums).
struct F32 {
  using elem = float;
  static constexpr const char* kName = "F32";
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
  // The V side of one super-block: the two V tiles in fragment order.
  template <int D>
  struct VPair {
    Frag<D> a, b;
  };
  template <int D>
  __device__ static void load_vpair(VPair<D>& v, const elem* va_tile, const elem* vb_tile, int lane) {
    load_tile(v.a, va_tile, lane);
    load_tile(v.b, vb_tile, lane);
  }
  template <int D>
  __device__ static void lds_vpair(VPair<D>& v, uint32_t va_addr, int lane) {
    load_tile_lds(v.a, va_addr, lane);
    load_tile_lds(v.b, va_addr + 16 * D * 4, lane);
  }
  // full fp32 weights: pmax plays no part
  template <int D>
  __device__ static void pv(const VPair<D>& v, const float* p, float pmax, f32x4* acc, float& l) {
    l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v.a.v[dt][i], p[i], acc[dt], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(v.b.v[dt][i], p[4 + i], acc[dt], 0, 0, 0);
    }
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

// Writing a decode step's new tokens from the attention launch itself.
// Work unit w of one record (n tokens of one block) and KV head:
//   * the tokens open their block (slot 0): the whole tile is written, the
//     tokens in slots 0 .. n - 1 and zeros elsewhere; units [0, 2 NCH) are the
//     K then V chunks (kFresh);
//   * otherwise only the tokens, kPlain units each: unit i kPlain + u of token
//     slot + i is, for u < D / PC, the 16-byte K chunk holding
//     d = PC u .. PC u + PC - 1, else its V element d = u - D / PC (inside the
//     bf16 8-byte unit, or fp32 chunk, of tokens 4 (slot / 4) .. + 3).
// value() loads a unit's contents (so that several units' loads can be in
// flight together: it only loads, a bf16 V chunk of a whole tile as four raw
// 32-bit parts), store() arranges and writes them.
template <class P, int D>
struct TokUnits {
  using E = typename P::elem;
  static constexpr int EB = static_cast<int>(sizeof(E));
  using L = Layout<EB>;
  static constexpr int PC = L::kPerChunk;
  static constexpr int NCH = 16 * D / PC;
  static constexpr int kFresh = 2 * NCH;
  static constexpr int kPlain = D / PC + D;
  __device__ static int units(const NewTok& t) { return t.slot == 0 ? kFresh : t.n * kPlain; }
  __device__ static size_t tile(const NewTok& t, int h, int hkv) {
    return (static_cast<size_t>(t.blk) * hkv + h) * (16 * D);
  }
  __device__ static u32x4 value(const NewTokens& x, const NewTok& t, int h, int hkv, int w) {
    const E* sk = static_cast<const E*>(x.k) + (static_cast<size_t>(t.src) * hkv + h) * D;
    const E* sv = static_cast<const E*>(x.v) + (static_cast<size_t>(t.src) * hkv + h) * D;
    const size_t row = static_cast<size_t>(hkv) * D;  // one token's row
    if (t.slot == 0) {
      if (w < NCH) {
        // a K chunk is PC consecutive elements of one token's row: one load
        int tok, d;
        L::k_coord(w, 0, tok, d);
        if (tok >= t.n) return u32x4{0u, 0u, 0u, 0u};
        return *reinterpret_cast<const u32x4*>(sk + tok * row + d);
      }
      // a V chunk is element d (fp32), or elements d and d + 1 (bf16), of
      // four consecutive tokens: one load per token
      int tok0, d;
      L::v_coord(w - NCH, 0, tok0, d);
      uint32_t part[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        part[i] = 0u;
        if (tok0 + i < t.n) {
          if constexpr (EB == 2) part[i] = *reinterpret_cast<const uint32_t*>(sv + (tok0 + i) * row + d);
          else part[i] = __builtin_bit_cast(uint32_t, sv[(tok0 + i) * row + d]);
        }
      }
      return u32x4{part[0], part[1], part[2], part[3]};
    }
    const int i = w / kPlain, u = w - i * kPlain;
    if (u < D / PC) return *reinterpret_cast<const u32x4*>(sk + i * row + u * PC);
    u32x4 r{0u, 0u, 0u, 0u};
    const E e = sv[i * row + (u - D / PC)];
    __builtin_memcpy(&r, &e, sizeof(E));
    return r;
  }
  // NT: nontemporal stores, whose lines go out without staying dirty in L2
  // until the kernel's end (3 us of a decode step on the fork workload,
  // measured, where each wave writes its own tokens and waits for them only
  // before the super-block that reads them); plain stores where the writers
  // wait for their acknowledgement at once
  template <bool NT, class T>
  __device__ static void put(T v, T* p) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
  }
  template <bool NT = true>
  __device__ static void store(const NewTokens& x, const NewTok& t, int h, int hkv, int w, const u32x4& v) {
    const size_t tl = tile(t, h, hkv);
    E* kt = static_cast<E*>(x.kpool) + tl;
    E* vt = static_cast<E*>(x.vpool) + tl;
    if (t.slot == 0) {
      if (w < NCH) {
        put<NT>(v, reinterpret_cast<u32x4*>(kt + w * PC));
      } else if constexpr (EB == 2) {
        // the raw parts hold elements d, d + 1 of tokens tok0 .. tok0 + 3; the
        // chunk is d of the four tokens, then d + 1 of them
        const u32x4 c{(v[0] & 0xffffu) | (v[1] << 16), (v[2] & 0xffffu) | (v[3] << 16),
                      (v[0] >> 16) | (v[1] & 0xffff0000u), (v[2] >> 16) | (v[3] & 0xffff0000u)};
        put<NT>(c, reinterpret_cast<u32x4*>(vt + (w - NCH) * PC));
      } else {
        put<NT>(v, reinterpret_cast<u32x4*>(vt + (w - NCH) * PC));
      }
      return;
    }
    const int i = w / kPlain, u = w - i * kPlain;
    const int slot = t.slot + i;
    if (u < D / PC) {
      int ch;
      if constexpr (EB == 2) ch = u * 16 + slot;
      else ch = (u >> 2) * 64 + (u & 3) * 16 + slot;
      put<NT>(v, reinterpret_cast<u32x4*>(kt + ch * PC));
    } else {
      const int d = u - D / PC;
      E e;
      __builtin_memcpy(&e, &v, sizeof(E));
      put<NT>(e, vt + ((d >> 4) * 64 + (slot >> 2) * 16 + (d & 15)) * 4 + (slot & 3));
    }
  }
};

// Whole tiles of up to four token records that open their blocks (slot 0),
// for KV heads [h0, h0 + NH), by NTH threads together, every load of every
// record in flight before the first store:
//   * K: job j is piece j % PR (PC consecutive elements) of token row
//     (j / PR) % 16 of head h0 + j / (16 PR), PR = D / PC: one 16-byte load,
//     16 lanes reading one token's row, then a store to the piece's chunk of
//     the tile;
//   * V: job j is chunk j % NCH of head h0 + j / NCH: element d (fp32), or
//     elements d and d + 1 (bf16), of four consecutive tokens, four 32-bit
//     loads.
// A row past the record's tokens is read from its last token and zeroed
// (no branch per chunk: the compiler waited for the loads at each join).
template <class P, int D, int NTH, int NH, bool NT>
__device__ void write_fresh_tiles(const NewTokens& x, const NewTok* t, int nt, int h0, int hkv, int tid) {
  using TU = TokUnits<P, D>;
  using E = typename P::elem;
  constexpr int EB = TU::EB;
  using L = typename TU::L;
  constexpr int PC = TU::PC, NCH = TU::NCH, PR = D / PC;
  constexpr int JOBS = NH * NCH;  // per kind (K or V) and record
  constexpr int JPT = (JOBS + NTH - 1) / NTH;
  constexpr int MAXT = 4;
  const size_t row = static_cast<size_t>(hkv) * D;
  u32x4 kp[MAXT][JPT];
  uint32_t vp[MAXT][JPT][4];
#pragma unroll
  for (int r = 0; r < MAXT; ++r) {
    if (r >= nt) break;
#pragma unroll
    for (int q = 0; q < JPT; ++q) {
      const int j = tid + q * NTH;
      if (JOBS % NTH != 0 && j >= JOBS) break;
      const int h = h0 + j / NCH, c = j % NCH;
      const E* kb = static_cast<const E*>(x.k) + (static_cast<size_t>(t[r].src) * hkv + h) * D;
      const E* vb = static_cast<const E*>(x.v) + (static_cast<size_t>(t[r].src) * hkv + h) * D;
      const int ktok = c / PR, piece = c % PR;
      kp[r][q] = *reinterpret_cast<const u32x4*>(kb + min(ktok, t[r].n - 1) * row + piece * PC);
      int tok, d;
      L::v_coord(c, 0, tok, d);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        vp[r][q][i] = *reinterpret_cast<const uint32_t*>(vb + min(tok + i, t[r].n - 1) * row + d);
    }
  }
  // every load issued before the first store
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int r = 0; r < MAXT; ++r) {
    if (r >= nt) break;
#pragma unroll
    for (int q = 0; q < JPT; ++q) {
      const int j = tid + q * NTH;
      if (JOBS % NTH != 0 && j >= JOBS) break;
      const int h = h0 + j / NCH, c = j % NCH;
      const size_t tl = TU::tile(t[r], h, hkv);
      // K: piece `piece` of token ktok is chunk (piece, ktok) of the tile
      const int ktok = c / PR, piece = c % PR;
      int kch;
      if constexpr (EB == 2) kch = piece * 16 + ktok;
      else kch = (piece >> 2) * 64 + (piece & 3) * 16 + ktok;
      const u32x4 kv = ktok < t[r].n ? kp[r][q] : u32x4{0u, 0u, 0u, 0u};
      TU::template put<NT>(kv, reinterpret_cast<u32x4*>(static_cast<E*>(x.kpool) + tl + kch * PC));
      int tok, d;
      L::v_coord(c, 0, tok, d);
      uint32_t p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = tok + i < t[r].n ? vp[r][q][i] : 0u;
      u32x4 v;
      if constexpr (EB == 2) {
        // the parts hold elements d, d + 1 of the four tokens; the chunk is d
        // of the four tokens, then d + 1 of them
        v = u32x4{(p[0] & 0xffffu) | (p[1] << 16), (p[2] & 0xffffu) | (p[3] << 16), (p[0] >> 16) | (p[1] & 0xffff0000u),
                  (p[2] >> 16) | (p[3] & 0xffff0000u)};
      } else {
        v = u32x4{p[0], p[1], p[2], p[3]};
      }
      TU::template put<NT>(v, reinterpret_cast<u32x4*>(static_cast<E*>(x.vpool) + tl + c * PC));
    }
  }
}

// The decode step's new tokens in this work item's blocks (DevItem::tails, at
// most 64), written by the whole workgroup (NTH threads) for its KV heads
// [h0, h0 + NH) before any of its threads reads the pool or the plan's block
// entries: the tiles (a block the tokens open whole, with zeros after them)
// and each block's valid count in the plan (every KV head's workgroup writes
// the same value).  Each wave holds the item's token records in its lanes
// (one load); whole tiles go four records at a time (write_fresh_tiles), the
// units of records in partly filled blocks four records at a time spread over
// the threads, with all their loads in flight together.  Only this workgroup
// reads these tiles and entries in the launch: an unfrozen tip block appears
// once in a plan.
template <class P, int D, int NTH, int NH>
__device__ void write_new_tokens(const NewTokens& x, const DevItem& it, int h0, int hkv, int tid) {
  using TU = TokUnits<P, D>;
  constexpr int nh = NH, nthreads = NTH;
  const int tk0 = it.tails & 0xffff, tkc = it.tails >> 16;
  if (tkc == 0) return;
  const int lane = tid & 63;
  int te = -1, tbk = 0, ts = 0, tn = 0, tsr = 0;
  if (lane < tkc && tk0 + lane < x.n) {
    const NewTok t = x.tok[tk0 + lane];
    te = t.entry;
    tbk = t.blk;
    ts = t.slot;
    tn = t.n;
    tsr = t.src;
  }
  auto rec = [&](int i) {
    return NewTok{__builtin_amdgcn_readlane(te, i), __builtin_amdgcn_readlane(tbk, i),
                  static_cast<int16_t>(__builtin_amdgcn_readlane(ts, i)),
                  static_cast<int16_t>(__builtin_amdgcn_readlane(tn, i)), __builtin_amdgcn_readlane(tsr, i)};
  };
  constexpr int MAXT = 4;
  uint64_t whole = __ballot(te >= 0 && ts == 0);
  uint64_t todo = __ballot(te >= 0 && ts != 0);
  if (!whole && !todo) return;
  while (whole) {
    NewTok t[MAXT];
    int nt = 0;
#pragma unroll
    for (int j = 0; j < MAXT; ++j) {
      t[j] = NewTok{-1, 0, 0, 0, 0};
      if (whole) {
        t[j] = rec(__builtin_ctzll(whole));
        whole &= whole - 1;
        nt = j + 1;
      }
    }
    write_fresh_tiles<P, D, NTH, NH, false>(x, t, nt, h0, hkv, tid);
#pragma unroll
    for (int j = 0; j < MAXT; ++j)  // (unrolled: a runtime index would put t on the stack)
      if (j < nt && tid == 0) x.blocks[t[j].entry].valid = t[j].slot + t[j].n;
  }
  while (todo) {
    NewTok t[MAXT];
    int nt = 0;
#pragma unroll
    for (int j = 0; j < MAXT; ++j) {
      t[j] = NewTok{-1, 0, 0, 0, 0};
      if (todo) {
        t[j] = rec(__builtin_ctzll(todo));
        todo &= todo - 1;
        nt = j + 1;
      }
    }
    // units of these records, thread-strided; a thread's share of a
    // one-token record's units is at most ceil(nh * units / nthreads) <= 4
    // for every shape here (the rest, below)
    constexpr int R = 4;
    u32x4 v[MAXT][R];
#pragma unroll
    for (int j = 0; j < MAXT; ++j) {
      if (j >= nt) break;
      const int per = TU::units(t[j]), total = nh * per;
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const int u = tid + k * nthreads;
        if (u < total) v[j][k] = TU::value(x, t[j], h0 + u / per, hkv, u % per);
      }
    }
#pragma unroll
    for (int j = 0; j < MAXT; ++j) {
      if (j >= nt) break;
      const int per = TU::units(t[j]), total = nh * per;
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const int u = tid + k * nthreads;
        if (u < total) TU::template store<false>(x, t[j], h0 + u / per, hkv, u % per, v[j][k]);
      }
      // a thread past R * nthreads units: the rest of this record, one at a time
      for (int u = tid + R * nthreads; u < total; u += nthreads)
        TU::template store<false>(x, t[j], h0 + u / per, hkv, u % per,
                                  TU::value(x, t[j], h0 + u / per, hkv, u % per));
      if (tid == 0) x.blocks[t[j].entry].valid = t[j].slot + t[j].n;
    }
  }
  // every store of the workgroup acknowledged (in L2) before any wave loads
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

}  // namespace attn
}  // namespace tkv
