// Shared device-side definitions for the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mask_engine.h"

namespace sdpa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// Problem description passed by value to every kernel.
struct KArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* d_o;
  const float* lse;
  const float* softmax_offset;  // [Hq] raw sink logits (learnable)
  const int32_t* seqlens;       // [B] or nullptr
  void* out_o;                  // forward output O
  float* out_lse;               // forward output LSE
  void* dq;
  void* dk;
  void* dv;
  float* delta;       // workspace [B,Hq,S]: rowsum(dO * O)
  float* lse2;        // workspace [B,Hq,S]: LSE * log2(e), 0 past the valid length
  float* dz_partial;  // workspace [B,Hq,nchunk]
  float* d_offset;    // [Hq] or nullptr
  int B, S, Hq, Hkv, G;
  int causal, wl, wr;   // windows already normalised to -1 or < S
  int softmax_type;     // 0 vanilla, 1 off-by-one, 2 learnable
  float scale;          // softmax scale on q.k
  float scale_log2;     // scale * log2(e)
  int n_tiles;          // tiles along the sequence for this kernel's grid
  int n_chunks;         // dz partial chunks per (b, h)
};

__device__ __forceinline__ int seq_len(const KArgs& a, int b) {
  int L = a.seqlens ? a.seqlens[b] : a.S;
  return L < 0 ? 0 : (L > a.S ? a.S : L);
}

// Sink logit z_h in natural-log units, or -inf when there is none.
__device__ __forceinline__ float sink_logit(const KArgs& a, int h) {
  if (a.softmax_type == 1) return 0.0f;
  if (a.softmax_type == 2) return a.softmax_offset[h];
  return -__builtin_inff();
}

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of lane (l xor 32) combined with this lane's by a symmetric operation.
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Key (or query) offset, inside a 32-wide block, of element i of a 32x32
// MFMA accumulator held by a lane in half hf (= lane / 32).
__device__ __forceinline__ int acc_row(int i, int hf) { return (i >> 2) * 8 + hf * 4 + (i & 3); }

// Position, inside a 16-wide step, where the operand that pairs with
// accumulator-derived values stores physical offset r: the accumulator of
// half hf holds rows {0-3, 8-11} (hf=0) or {4-7, 12-15} (hf=1) of each 16,
// so groups of four rows 1 and 2 trade places.
__device__ __forceinline__ int perm16(int r) {
  const int g = (r >> 2) & 3;
  const int pg = (g == 1) ? 2 : (g == 2 ? 1 : g);
  return (r & ~15) + pg * 4 + (r & 3);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Raw buffer resource over [base, base + bytes): loads at or past the end
// return zero, so padded rows read as zeros without per-lane branches.
// Word 3 (0x00020000) selects 32-bit data format for raw (untyped) access.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

// A operand (rows = head dims, reduction = sequence positions) of a 32x32x16
// MFMA, read with two LDS transpose loads from a row-major [position][dim]
// bf16 tile.  Within each 16-lane group the transpose load treats the 8-byte
// chunks of lanes 4s..4s+3 as row s of a 4x16 matrix and hands lane c
// its column c.  Lane l (group G = l/16, half hf = G/2) therefore addresses
// position pos0 + hf*4 + s at dims d0 + (G%2)*16 + 4q (s = (l/4)%4, q = l%4)
// and receives dim d0 + l%32 of positions pos0 + hf*4 + {0..3}; the second
// load adds 8 positions.  Those are exactly the rows acc_row(e, hf), e = 0..7,
// that a lane of a 32x32 accumulator holds for the same 16 positions, so the
// B operand can come straight from accumulator registers.
__device__ __forceinline__ bf16x8 lds_tr_operand(const uint16_t* tile, int pitch, int pos0, int d0, int lane) {
  const int G = lane >> 4, s = (lane >> 2) & 3, q = lane & 3;
  const uint16_t* p = tile + (pos0 + (G >> 1) * 4 + s) * pitch + d0 + (G & 1) * 16 + q * 4;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * pitch));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}

// ---- swizzled row-major bf16 tiles in LDS ---------------------------------
//
// A tile holds R rows of CH 16-byte chunks with no padding; logical chunk c
// of row r is stored at physical chunk c ^ swz(r).  With 64 four-byte banks
// (256 B per cycle) the two read patterns the kernels use are then free of
// bank conflicts:
//   row reads  (ds_read_b128): 16 lanes read one chunk of 16 consecutive rows;
//   transpose loads (lds_tr): 32 lanes read 4 chunks of 4 consecutive rows.
// 256-byte rows all start on bank 0, so swz must spread 16 consecutive rows
// over 16 distinct chunks and 4 consecutive rows over 4 distinct chunk
// quads; 128- and 384-byte rows alternate between the two 128-byte halves of
// the bank array, so swz (kept below 8, which keeps c ^ swz inside the row)
// must do the same for every other row.  swz is a bijection on the rows of
// any aligned group of 16 in both cases.
template <int CH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CH == 16) return 4 * (r & 3) + ((r >> 2) & 3);
  else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}
template <int CH>
__device__ __forceinline__ int swz_off(int r, int c) { return (r * CH + (c ^ swz<CH>(r))) * 16; }

// 16-byte row read of logical chunk c of row r.
template <int CH>
__device__ __forceinline__ u32x4 tile_row16(const uint16_t* tile, int r, int c) {
  return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(tile) + swz_off<CH>(r, c));
}

// lds_tr_operand for a swizzled tile (dims d0 .. d0+31, positions pos0 .. pos0+15).
template <int CH>
__device__ __forceinline__ bf16x8 tile_tr_operand(const uint16_t* tile, int pos0, int d0, int lane) {
  const int G = lane >> 4, s = (lane >> 2) & 3, q = lane & 3;
  const int row = pos0 + (G >> 1) * 4 + s;
  const int dim = d0 + (G & 1) * 16 + q * 4;
  const char* base = reinterpret_cast<const char*>(tile) + (dim & 7) * 2;
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + swz_off<CH>(row, dim >> 3)));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + swz_off<CH>(row + 8, dim >> 3)));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
}

// Asynchronous copy of rows [row0, row0 + R) of a row-major bf16 tensor
// (rows `stride_bytes` apart, starting at the buffer resource's base) into a
// swizzled LDS tile, straight from memory to LDS (no registers).  Each
// instruction moves 64 consecutive physical chunks: lane l of the wave fills
// physical chunk idx = base + l, i.e. row idx / CH, logical chunk
// (idx % CH) ^ swz(row).  Rows past the resource's end arrive as zeros.
// Complete with lds_dma_wait() and a workgroup barrier before reading.
template <int R, int CH, int NT>
__device__ __forceinline__ void tile_dma(__amdgpu_buffer_rsrc_t res, uint32_t stride_bytes, int row0,
                                         uint16_t* tile, int tid) {
  static_assert((R * CH) % (NT) == 0, "tile must split into whole wave instructions");
  constexpr int PER_WAVE = R * CH / NT;  // instructions per wave
  const int w = tid >> 6, lane = tid & 63;
  typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
  for (int k = 0; k < PER_WAVE; ++k) {
    const int base = (w * PER_WAVE + k) * 64;
    const int idx = base + lane;
    const int row = idx / CH, c = (idx % CH) ^ swz<CH>(row);
    const uint32_t voff = (uint32_t)(row0 + row) * stride_bytes + (uint32_t)c * 16;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (lds_void*)(reinterpret_cast<char*>(tile) + base * 16), 16, voff,
                                             0, 0, 0);
  }
}

__device__ __forceinline__ void lds_dma_wait() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Keys visible from query row qi, as an inclusive interval [lo, hi]
// (empty when lo > hi).  Same rule as visible(): row qi < L sees keys
// max(0, qi-wl) .. min(L-1, qi [causal], qi+wr).
__device__ __forceinline__ void row_key_bounds(const MaskSpec& m, int qi, int& lo, int& hi) {
  lo = m.wl >= 0 ? (qi - m.wl > 0 ? qi - m.wl : 0) : 0;
  hi = m.L - 1;
  if (m.causal && qi < hi) hi = qi;
  if (m.wr >= 0 && qi + m.wr < hi) hi = qi + m.wr;
  if (qi >= m.L) { lo = 1; hi = 0; }
}

// Query rows that see key kj, as an inclusive interval [lo, hi]: the same
// rule read by column, rows max(0, kj [causal], kj-wr) .. min(L-1, kj+wl).
__device__ __forceinline__ void col_query_bounds(const MaskSpec& m, int kj, int& lo, int& hi) {
  lo = 0;
  if (m.causal) lo = kj;
  if (m.wr >= 0 && kj - m.wr > lo) lo = kj - m.wr;
  hi = m.L - 1;
  if (m.wl >= 0 && kj + m.wl < hi) hi = kj + m.wl;
  if (kj >= m.L) { lo = 1; hi = 0; }
}

}  // namespace sdpa
