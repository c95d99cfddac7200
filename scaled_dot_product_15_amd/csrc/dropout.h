// Attention dropout: keep decisions from the counter-based generator
// Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011), written from that definition.
//
// The TE single-GPU page ("Other attention knobs") turns attention dropout on
// with a rate and an RNG, and the forward of PR #2225's sequence diagrams
// hands back an rng_state; the generator and the layout below are this
// library's reading.  Pair (query row i, key j) of batch b and query head h
// is kept iff its random byte is at least t = round(256 p): one generator
// call covers the 4 x 4 block of pairs (i & ~3 .., j & ~3 ..) with counter
// (j >> 2, i >> 2, b * Hq + h, offset) and key (seed low word, seed high
// word); pair (i, j) takes byte (i & 3) * 4 + (j & 3) of the 16 output bytes
// (word byte / 4, bits 8 * (byte % 4) up).  Kept probabilities are scaled by
// 1 / (1 - t / 256) (inverted dropout); the softmax normalisation and the
// LSE use the undropped probabilities.
#pragma once

#include "attn_common.h"

namespace sdpa {

// Counter words c, key (k0, k1): ten rounds, each multiplying counter words 0
// and 2 by the round multipliers and mixing the product halves with words 1
// and 3 and the round key; the key advances by the Weyl increments between
// rounds.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    c = u32x4{(uint32_t)(p1 >> 32) ^ c[1] ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c[3] ^ k1, (uint32_t)p0};
  }
  return c;
}

// The generator state and threshold, copied out of the kernel arguments once
// (plain scalars, so they stay in scalar registers).
struct DropGen {
  uint32_t seed_lo, seed_hi, offset;
  int t;        // byte threshold; 0 = no dropout
  float scale;  // 1 / (1 - t / 256)
};
__device__ __forceinline__ DropGen drop_gen(const KArgs& a) {
  return DropGen{a.drop_seed_lo, a.drop_seed_hi, a.drop_offset, a.drop_t, a.drop_scale};
}

__device__ __forceinline__ u32x4 drop_block(const DropGen& d, int bh, int i, int j) {
  return philox4x32_10(u32x4{(uint32_t)j >> 2, (uint32_t)i >> 2, (uint32_t)bh, d.offset}, d.seed_lo, d.seed_hi);
}

// Random bytes of pairs (i, j4 + c), c = 0..3, as byte c of the result
// (j4 % 4 == 0): lanes that own a query row (forward, dQ).
// Word i & 3 is picked with AND / OR masks: a chain of selects on the
// lane-varying row would be turned into divergent branches.
__device__ __forceinline__ uint32_t drop_bytes_row(const DropGen& d, int bh, int i, int j4) {
  const u32x4 w = drop_block(d, bh, i, j4);
  const int r = i & 3;
  const uint32_t m0 = 0u - (uint32_t)(r == 0), m1 = 0u - (uint32_t)(r == 1), m2 = 0u - (uint32_t)(r == 2),
                 m3 = 0u - (uint32_t)(r == 3);
  return (w[0] & m0) | (w[1] & m1) | (w[2] & m2) | (w[3] & m3);
}

// Random bytes of pairs (i4 + r, j), r = 0..3, as byte r of the result
// (i4 % 4 == 0): lanes that own a key (dK / dV).
__device__ __forceinline__ uint32_t drop_bytes_col(const DropGen& d, int bh, int i4, int j) {
  const u32x4 w = drop_block(d, bh, i4, j);
  const uint32_t sh = (uint32_t)(j & 3) * 8;
  return ((w[0] >> sh) & 0xFFu) | (((w[1] >> sh) & 0xFFu) << 8) | (((w[2] >> sh) & 0xFFu) << 16) |
         (((w[3] >> sh) & 0xFFu) << 24);
}

// ---- one generator call per lane, shared across a lane quad ------------------
//
// In the kernels the four lanes of a quad (lanes 4m .. 4m+3) hold the four
// rows (forward, dQ) or the four keys (dK / dV) of the same 4 x 4 blocks, so
// they need the same calls.  Lane r of the quad makes only the call of group
// r and the quad exchanges the results: a 4 x 4 transpose across the quad
// (lane r holding row r of A ends up with column r), done as two butterfly
// stages of DPP quad permutes (partners r ^ 2, then r ^ 1), each stage
// swapping the two words whose index bit differs from the lane's.

// DPP quad_perm controls: lane r reads lane r ^ 2, resp. r ^ 1.
constexpr int kQuadSwap2 = 2 | (3 << 2) | (0 << 4) | (1 << 6);
constexpr int kQuadSwap1 = 1 | (0 << 2) | (3 << 4) | (2 << 6);

__device__ __forceinline__ uint32_t quad_read(uint32_t v, int ctrl_selector) {
  return ctrl_selector == 2
             ? (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kQuadSwap2, 0xF, 0xF, false)
             : (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kQuadSwap1, 0xF, 0xF, false);
}

// a[c] = A[r][c] on lane r (r = lane % 4) -> a[c] = A[c][r].
__device__ __forceinline__ void quad_transpose(uint32_t (&a)[4], int r) {
  const bool hi = (r & 2) != 0, lo = (r & 1) != 0;
#pragma unroll
  for (int p = 0; p < 2; ++p) {  // words p and p + 2 with lanes r ^ 2
    const uint32_t recv = quad_read(hi ? a[p] : a[p + 2], 2);
    a[p] = hi ? recv : a[p];
    a[p + 2] = hi ? a[p + 2] : recv;
  }
#pragma unroll
  for (int p = 0; p < 4; p += 2) {  // words p and p + 1 with lanes r ^ 1
    const uint32_t recv = quad_read(lo ? a[p] : a[p + 1], 1);
    a[p] = lo ? recv : a[p];
    a[p + 1] = lo ? a[p + 1] : recv;
  }
}

// Row lanes (query row i, i % 4 == lane % 4): out[g] = random bytes of pairs
// (i, jb + 8g + c), c = 0..3, for g = 0..3 (jb % 4 == 0); same as
// drop_bytes_row(d, bh, i, jb + 8g).
__device__ __forceinline__ void drop_rows_quad(const DropGen& d, int bh, int i, int jb, uint32_t (&out)[4]) {
  const int r = i & 3;
  const u32x4 w = drop_block(d, bh, i, jb + 8 * r);
  out[0] = w[0];
  out[1] = w[1];
  out[2] = w[2];
  out[3] = w[3];
  quad_transpose(out, r);
}

// Column lanes (key j, j % 4 == lane % 4): out[g] = random bytes of pairs
// (ib + 8g + r, j), r = 0..3, for g = 0..3 (ib % 4 == 0); same as
// drop_bytes_col(d, bh, ib + 8g, j).
__device__ __forceinline__ void drop_cols_quad(const DropGen& d, int bh, int ib, int j, uint32_t (&out)[4]) {
  const int c = j & 3;
  const u32x4 w = drop_block(d, bh, ib + 8 * c, j);
#pragma unroll
  for (int x = 0; x < 4; ++x) {  // column x of the call's 4 x 4 bytes
    const uint32_t sh = 8u * x;
    out[x] = ((w[0] >> sh) & 0xFFu) | (((w[1] >> sh) & 0xFFu) << 8) | (((w[2] >> sh) & 0xFFu) << 16) |
             (((w[3] >> sh) & 0xFFu) << 24);
  }
  quad_transpose(out, c);
}

// Byte n of a random word against the threshold.
__device__ __forceinline__ bool drop_keep(uint32_t bytes, int n, int t) {
  return (int)((bytes >> (8 * n)) & 0xFFu) >= t;
}

// Keep decision of one pair (any layout; the fp32 kernels and the debug export).
__device__ __forceinline__ bool drop_keep_pair(const DropGen& d, int bh, int i, int j) {
  return drop_keep(drop_bytes_row(d, bh, i, j & ~3), j & 3, d.t);
}

}  // namespace sdpa
