// Element order inside one pool tile: 16 token slots x D of one (layer, block, KV head).
//
// The tile is a sequence of 16-byte chunks.  The order is chosen so that load
// number i of lane L of a wave reads chunk i*64 + L: every wave load is one
// contiguous 1 KiB run of HBM, and the lane ends up holding exactly the MFMA
// operand fragment it needs, with no LDS transpose.
//
// bf16 (8 elements per chunk), lane L = 16*g + n:
//   K chunk c*16 + n, element e   = K[token n][d = 8c + e]            (c < D/8)
//     -> load i gives lane (g, n) K[n][32i + 8g + 0..7]: the A operand of a
//        16x16x32 MFMA computing S^T = K Q^T (rows = tokens).
//   V is kept in 8-byte units (half a chunk): unit u = dt*64 + g*16 + dl, element
//   i = V[token 4g + i][d = 16dt + dl]; chunk ch holds units 2ch and 2ch + 1
//     -> 8-byte load dt of lane (g, dl) reads unit dt*64 + L: V^T[d][tokens
//        4g..4g+3] for d = 16dt + dl, half of the A operand of the 16x16x32 MFMA
//        computing O^T += V^T P^T (the other half comes from the next block).
// fp32 (4 elements per chunk):
//   K chunk c*64 + g*16 + n, element e = K[token n][d = 16c + 4g + e]   (c < D/16)
//   V chunk t*64 + g*16 + dl, element e = V[token 4g + e][d = 16t + dl]  (t < D/16)
#pragma once

namespace tkv {

template <int ELEM_BYTES>
struct Layout;

template <>
struct Layout<2> {
  static constexpr int kPerChunk = 8;
  __device__ static inline void k_coord(int ch, int e, int& tok, int& d) {
    tok = ch & 15;
    d = 8 * (ch >> 4) + e;
  }
  __device__ static inline void v_coord(int ch, int e, int& tok, int& d) {
    const int u = 2 * ch + (e >> 2);
    const int dt = u >> 6, g = (u >> 4) & 3, dl = u & 15;
    tok = 4 * g + (e & 3);
    d = 16 * dt + dl;
  }
};

template <>
struct Layout<4> {
  static constexpr int kPerChunk = 4;
  __device__ static inline void k_coord(int ch, int e, int& tok, int& d) {
    const int c = ch >> 6, g = (ch >> 4) & 3;
    tok = ch & 15;
    d = 16 * c + 4 * g + e;
  }
  __device__ static inline void v_coord(int ch, int e, int& tok, int& d) {
    const int t = ch >> 6, g = (ch >> 4) & 3, dl = ch & 15;
    tok = 4 * g + e;
    d = 16 * t + dl;
  }
};

}  // namespace tkv
