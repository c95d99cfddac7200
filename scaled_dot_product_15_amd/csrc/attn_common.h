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
  const int32_t* seq_offsets;   // [B+1] segment starts of packed (THD) tensors, or nullptr (BSHD)
  void* out_o;                  // forward output O
  float* out_lse;               // forward output LSE
  void* dq;
  void* dk;
  void* dv;
  float* delta;       // workspace [B,Hq,S]: rowsum(dO * O)
  float* lse2;        // workspace [B,Hq,S]: LSE * log2(e), 0 past the valid length
  float* dz_partial;  // workspace [B,Hq,nchunk]
  float* kv_part;     // workspace [n_splits][B,S,Hkv,Dqk] then [n_splits][B,S,Hkv,Dv]: partial dK / dV
  float* d_offset;    // [Hq] or nullptr
  int B, S, Hq, Hkv, G;
  int causal, wl, wr;   // windows already normalised to -1 or < S
  int softmax_type;     // 0 vanilla, 1 off-by-one, 2 learnable
  float scale;          // softmax scale on q.k
  float scale_log2;     // scale * log2(e)
  int n_tiles;          // tiles along the sequence for this kernel's grid
  int n_chunks;         // dz partial chunks per (b, h)
  int n_splits;         // dK/dV workgroups per (key tile, batch, kv head), each over G / n_splits query heads
  const void* bias;     // additive post-scale bias [bias_b, bias_h, S, S] (bf16), or nullptr
  void* d_bias;         // its gradient, same shape, or nullptr
  int bias_b, bias_h;   // 1 (shared) or B / Hq
  float inv_scale;      // 1 / scale: the kernels add bias / scale to the unscaled scores
  const float* fp8_descale;  // FP8: descales of Q, K, V (and dO in the backward), device
  uint8_t* vt;          // FP8 forward workspace: V^T [B, Hkv, Dv, S_pad] with permuted key order
  uint8_t* kt_t;        // FP8 backward workspace: K^T [B, Hkv, D, S_pad], permuted key order
  uint8_t* qt_t;        //   Q^T [B, Hq, D, S_pad], permuted row order
  uint8_t* dot_t;       //   dO^T [B, Hq, Dv, S_pad], permuted row order
  const float* ds_scale;  // FP8 backward: per-tensor scale of dS before its E5M2 encoding (device, [1])
  float* amax_out;      // FP8 backward: max |dS| (device, [1]; cleared by the launcher)
  int s_pad;            // S rounded up to the FP8 key tile (64)
  int dbias_direct;     // bias not shared (B x Hq matrices): the dQ kernel writes dBias = dS itself
  int drop_t;           // dropout byte threshold round(256 p); 0 = no dropout
  float drop_scale;     // 1 / (1 - drop_t / 256)
  uint32_t drop_seed_lo, drop_seed_hi, drop_offset;  // generator key and counter word 3
  // bf16 backward with stored dS: the dK/dV kernel writes its bf16 dS blocks
  // here and the dQ kernel reads them instead of recomputing S and dP
  // (nullptr: dQ recomputes).  Per (batch, query head) ds_head_blocks blocks
  // of 32 rows x 128 keys (8 KiB): the slabs of the 128-key tiles in order,
  // ds_tile_blocks(kt) blocks each, block r of a slab holding the rows
  // q_first + 32 r .. +31, q_first the tile's first visible row rounded down
  // to a multiple of 64.
  uint16_t* ds;
  int ds_head_blocks;
};

// Workgroup order of the bf16 kernels (q_tile_of, the dK/dV kernel): for head
// dims of 128 and up the items that share K / V (or Q / dO) rows are grouped
// on one XCD, where those rows are large (measured per step: GQA+SWA S=4096
// 2-5 %, MLA 192/128 10 %, sink + padding S=8192 4 % faster); the 64-dim
// kernels keep the heaviest tiles first over the whole grid (the 64-dim
// sweep's short sequences ran 10 % slower grouped).
template <int DQK>
constexpr bool kGroupedOrder = DQK >= 128;

// Sign of the stored dS blocks: the dK/dV kernel stores the B operand of its
// dK products, which is -dS where delta is folded into its dP products (no
// dropout) and dS with dropout.
__device__ __forceinline__ float ds_stored_sign(const KArgs& a) { return a.drop_t > 0 ? 1.0f : -1.0f; }

// Stored-dS slab of key tile kt: its first block within the (batch, head)
// region and its block count, from the mask at the full length S (a loop over
// the tiles before it: a few scalar instructions each, once per workgroup).
__device__ __forceinline__ void ds_slab(const KArgs& a, int kt, int& first, int& count) {
  const MaskSpec mf = make_mask(a.S, a.S, a.causal, a.wl, a.wr);
  first = 0;
  for (int t = 0; t < kt; ++t) first += ds_tile_blocks(mf, t);
  count = ds_tile_blocks(mf, kt);
}

// Group and item of workgroup `id` in a grid of n_groups x per_group work
// items where the items of one group read the same rows (the K tiles of a KV
// head, the Q / dO rows of a key tile's neighbours): the hardware deals
// consecutive workgroups round-robin over the 8 XCDs, each with its own L2, so
// group n's items go to XCD n % 8 in consecutive slots there and run at the
// same time, sharing that L2.  Groups past the last multiple of 8 are dealt
// in plain order.  A bijection of [0, n_groups * per_group).
__device__ __forceinline__ void xcd_group_item(int id, int n_groups, int per_group, int& group, int& item) {
  const int full = (n_groups / 8) * 8 * per_group;
  if (id < full) {
    const int xcd = id & 7, slot = id >> 3;
    group = (slot / per_group) * 8 + xcd;
    item = slot % per_group;
  } else {
    group = id / per_group;
    item = id % per_group;
  }
}

// Query tile, batch and head of workgroup `id` of the forward and dQ kernels
// (n_tiles query tiles per head).  Grouped order: the G heads x n_tiles tiles
// of a (batch, KV head) read the same K / V tiles, so they run together on
// one XCD (xcd_group_item), heaviest query tiles first (the last ones under a
// causal mask) and the G heads of a tile side by side.  Otherwise the
// heaviest tiles of every head come first over the whole grid (the tail is
// balanced best) and only the G heads of a tile share an XCD.
template <bool GROUPED>
__device__ __forceinline__ void q_tile_of(const KArgs& a, int id, int& b, int& h, int& qt) {
  if constexpr (GROUPED) {
    int grp, item;
    xcd_group_item(id, a.B * a.Hkv, a.G * a.n_tiles, grp, item);
    b = grp / a.Hkv;
    const int g = grp % a.Hkv;
    qt = a.n_tiles - 1 - item / a.G;
    h = g * a.G + item % a.G;
  } else {
    // the G heads of one query tile on consecutive ids of one XCD
    const int N = a.B * a.Hq * a.n_tiles, chunk = a.G, full = (N / (8 * chunk)) * (8 * chunk);
    int l = id;
    if (l < full) {
      const int xcd = l & 7, slot = l >> 3;
      l = ((slot / chunk) * 8 + xcd) * chunk + slot % chunk;
    }
    const int per_tile = a.B * a.Hq;
    qt = a.n_tiles - 1 - l / per_tile;
    b = (l % per_tile) / a.Hq;
    h = (l % per_tile) % a.Hq;
  }
}

// First row of batch b along the token axis of Q, K, V, O and the gradients:
// b * S for BSHD tensors; the start of segment b for packed (THD) tensors.
__device__ __forceinline__ size_t seq_row0(const KArgs& a, int b) {
  return a.seq_offsets ? (size_t)a.seq_offsets[b] : (size_t)b * a.S;
}

// Rows batch b owns along that axis: S (BSHD) or the size of segment b
// (THD), clamped to [0, S].  Kernels write output rows below this count only.
__device__ __forceinline__ int seq_rows(const KArgs& a, int b) {
  if (!a.seq_offsets) return a.S;
  const int n = a.seq_offsets[b + 1] - a.seq_offsets[b];
  return n < 0 ? 0 : (n > a.S ? a.S : n);
}

// Valid (unpadded) length of batch b, clamped to [0, seq_rows(a, b)].
__device__ __forceinline__ int seq_len(const KArgs& a, int b) {
  const int R = seq_rows(a, b);
  const int L = a.seqlens ? a.seqlens[b] : R;
  return L < 0 ? 0 : (L > R ? R : L);
}

// The [S, S] bias matrix of batch b, query head h: the [bias_b, bias_h, S, S]
// tensor with its size-1 dims broadcast.
__device__ __forceinline__ const uint16_t* bias_matrix(const KArgs& a, int b, int h) {
  const int bb = a.bias_b == 1 ? 0 : b, hh = a.bias_h == 1 ? 0 : h;
  return static_cast<const uint16_t*>(a.bias) + ((size_t)bb * a.bias_h + hh) * a.S * a.S;
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

// FP8 transposed tiles ([dims][positions], 64 positions per group): slot of
// position k (0..63) of a group.  Half hf of a 64-byte row holds the
// positions a lane of half hf holds in two 32x32 accumulator blocks, byte
// 16 kb + e for position 32 kb + acc_row(e, hf), so an accumulator-side
// operand of the 32x32x64 FP8 MFMA (one byte per element, packed in element
// order) pairs byte for byte with a 32-byte read of that half.
__host__ __device__ __forceinline__ int fp8_key_slot(int k) {
  const int kb = k >> 5, r = k & 31;
  const int hf = (r >> 2) & 1, e = (r >> 3) * 4 + (r & 3);
  return hf * 32 + kb * 16 + e;
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
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0));
}

// The two bf16 halves of a 32-bit word as floats (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Bias of one query row for the keys a lane holds in a 32x32 accumulator
// whose column is that row (forward, dQ: lane = query): element 4g + e of
// block kb is key j0 + kb*32 + g*8 + hf*4 + e, i.e. four runs of four
// consecutive keys, one 8-byte load each.  The resource spans the row's
// [S, S] matrix: keys past the row end read the next row (masked pairs) and
// nothing past the matrix is read.
template <int NKB>
struct RowBias {
  __amdgpu_buffer_rsrc_t res;
  uint32_t off;  // byte offset of (row, hf*4)
  u32x2 w[NKB][4];
  __device__ __forceinline__ void init(const KArgs& a, int b, int h, int qi, int hf) {
    res = buf_rsrc(bias_matrix(a, b, h), (uint32_t)((size_t)a.S * a.S * 2));
    const int row = qi < a.S ? qi : a.S - 1;  // rows past S are masked
    off = (uint32_t)((size_t)row * a.S + hf * 4) * 2;
  }
  __device__ __forceinline__ void load(int j0) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) w[kb][g] = buf_load8(res, off + (uint32_t)(j0 + kb * 32 + g * 8) * 2);
  }
  // s += bias * inv_scale on element 4g + e of block kb.
  __device__ __forceinline__ void add(f32x16 (&s)[NKB], float inv_scale) const {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        s[kb][4 * g + 0] = fmaf(bf16_lo(w[kb][g][0]), inv_scale, s[kb][4 * g + 0]);
        s[kb][4 * g + 1] = fmaf(bf16_hi(w[kb][g][0]), inv_scale, s[kb][4 * g + 1]);
        s[kb][4 * g + 2] = fmaf(bf16_lo(w[kb][g][1]), inv_scale, s[kb][4 * g + 2]);
        s[kb][4 * g + 3] = fmaf(bf16_hi(w[kb][g][1]), inv_scale, s[kb][4 * g + 3]);
      }
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

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
// 64-byte rows (CH == 4, the FP8 tiles) put four rows on the bank array, so
// swz spreads the four rows of each group of 16 that share a bank quarter
// over the four chunks.
template <int CH>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CH == 16) return 4 * (r & 3) + ((r >> 2) & 3);
  else if constexpr (CH == 4) return (r >> 2) & 3;
  else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}
template <int CH>
__device__ __forceinline__ int swz_off(int r, int c) { return (r * CH + (c ^ swz<CH>(r))) * 16; }

// Wave index within the workgroup, marked wave-uniform so that everything
// derived from it (row offsets, mask tile classes, LDS destinations) stays in
// scalar registers.
__device__ __forceinline__ int wave_id(int tid) { return __builtin_amdgcn_readfirstlane(tid >> 6); }

// ---- direct memory -> LDS copies -------------------------------------------
//
// buffer_load ... lds writes lane l's dwords to LDS address M0 + size * l
// without touching registers.  The copies are issued from inline assembly:
// the compiler then does not track them, and so does not put a wait for all
// outstanding copies in front of every LDS transpose load (it cannot tell
// that those read the other buffer).  Completion is therefore the caller's
// job: lds_dma_wait() and a workgroup barrier before any wave reads the
// destination.  The resource is a raw buffer over [base, base + bytes):
// lanes whose offset reaches past the end receive zeros.
struct BufDesc {
  u32x4 w;  // base lo, base hi (stride 0), byte count, raw 32-bit format
};
__device__ __forceinline__ BufDesc buf_desc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return BufDesc{u32x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xffffu, bytes, 0x00020000u}};
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  typedef __attribute__((address_space(3))) const char lds_char;
  return (uint32_t)reinterpret_cast<uintptr_t>((lds_char*)p);
}
// The resource and the LDS address are wave-uniform by construction;
// readfirstlane states it, so they are always in scalar registers as the
// instruction requires (it folds away where the compiler already knows).
__device__ __forceinline__ u32x4 uniform4(u32x4 v) {
  return u32x4{(uint32_t)__builtin_amdgcn_readfirstlane((int)v[0]), (uint32_t)__builtin_amdgcn_readfirstlane((int)v[1]),
               (uint32_t)__builtin_amdgcn_readfirstlane((int)v[2]), (uint32_t)__builtin_amdgcn_readfirstlane((int)v[3])};
}
// M0 is written here and nowhere else in these kernels; the hardware needs
// one wait state between the M0 write and the copy that reads it.
__device__ __forceinline__ void lds_dma16(const BufDesc& d, uint32_t lds_dst, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds_dst)), "v"(voff), "s"(uniform4(d.w))
               : "memory", "m0");
}
// The same copy with the non-temporal cache policy, for data read once
// (streamed blocks that should not displace reused tiles in L2).
__device__ __forceinline__ void lds_dma16_nt(const BufDesc& d, uint32_t lds_dst, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds_dst)), "v"(voff), "s"(uniform4(d.w))
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const BufDesc& d, uint32_t lds_dst, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"((uint32_t)__builtin_amdgcn_readfirstlane((int)lds_dst)), "v"(voff), "s"(uniform4(d.w))
               : "memory", "m0");
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt fields at their no-wait maxima),
// issued through the builtin so the compiler sees it and counts every
// earlier memory load of its own as complete from here on.
__device__ __forceinline__ void lds_dma_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---- reads of swizzled tiles -----------------------------------------------
//
// Loop-invariant per-lane byte offsets, so each LDS read in a hot loop is
// "lane offset + immediate" with no address arithmetic.  swz depends on the
// row modulo 16 only, so offsets computed for the first rows hold for every
// row block that starts on a multiple of 16; only the immediate changes.

// 16-byte row reads (B or A operand of a contraction over head dims): lane l
// reads row rb + l%32, logical chunk 2*ks + l/32, i.e. dims [16 ks + 8 (l/32), +8).
template <int CH>
struct RowReads {
  uint32_t off[CH / 2];
  __device__ __forceinline__ explicit RowReads(int lane) {
    const int r = lane & 31, hf = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < CH / 2; ++ks) off[ks] = (uint32_t)(r * CH + ((2 * ks + hf) ^ swz<CH>(r))) * 16;
  }
  // rb: first row of the 32-row block (a multiple of 32).
  __device__ __forceinline__ u32x4 read(const uint16_t* tile, int rb, int ks) const {
    return *reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(tile) + rb * CH * 16 + off[ks]);
  }
};

// A operand (rows = head dims, reduction = sequence positions) of a 32x32x16
// MFMA, read with two LDS transpose loads from a row-major [position][dim]
// tile.  Within each 16-lane group the transpose load treats the 8-byte
// chunks of lanes 4s..4s+3 as row s of a 4x16 matrix and hands lane c its
// column c.  Lane l (group G = l/16, half hf = G/2) therefore addresses
// position pos0 + hf*4 + s at dims d0 + (G%2)*16 + 4q (s = (l/4)%4, q = l%4)
// and receives dim d0 + l%32 of positions pos0 + hf*4 + {0..3}; the second
// load adds 8 positions.  Those are exactly the rows acc_row(e, hf), e = 0..7,
// that a lane of a 32x32 accumulator holds for the same 16 positions, so the
// B operand can come straight from accumulator registers.  db selects the
// 32-dim block d0 = 32 db.
template <int CH>
struct TrReads {
  static constexpr int NDB = CH / 4;
  uint32_t off[2][NDB];
  __device__ __forceinline__ explicit TrReads(int lane) {
    const int G = lane >> 4, s = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int row = (G >> 1) * 4 + s + 8 * h, dim = db * 32 + (G & 1) * 16 + q * 4;
        off[h][db] = (uint32_t)(swz_off<CH>(row, dim >> 3) + (dim & 7) * 2);
      }
  }
  // pos0: first of the 16 positions (a multiple of 16).
  __device__ __forceinline__ bf16x8 read(const uint16_t* tile, int pos0, int db) const {
    const char* t = reinterpret_cast<const char*>(tile) + pos0 * CH * 16;
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + off[0][db]));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + off[1][db]));
    const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
    return as_bf16x8(u32x4{a[0], a[1], b[0], b[1]});
  }
};

// Copy of rows [row0, row0 + R) of a row-major bf16 tensor (rows
// stride_bytes apart) into a swizzled LDS tile.  Each wave instruction moves
// 64 consecutive physical chunks: lane l fills physical chunk idx = base + l,
// i.e. row idx / CH, logical chunk (idx % CH) ^ swz(row).  The resource of
// each copy starts at row0 and ends at the valid length, so the per-lane
// source offsets never change and rows past the end arrive as zeros.
template <int R, int CH, int NT>
struct TileCopy {
  static_assert((R * CH) % NT == 0, "tile must split into whole wave instructions");
  static constexpr int PER_WAVE = R * CH / NT;
  uint32_t voff[PER_WAVE];
  int chunk0;  // first physical chunk this wave fills
  __device__ __forceinline__ TileCopy(int tid, uint32_t stride_bytes) {
    const int w = wave_id(tid), lane = tid & 63;
    chunk0 = w * PER_WAVE * 64;
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) {
      const int idx = chunk0 + k * 64 + lane;
      const int row = idx / CH, c = (idx % CH) ^ swz<CH>(row);
      voff[k] = (uint32_t)row * stride_bytes + (uint32_t)c * 16;
    }
  }
  // Rows [row0, row0 + R) from a resource of `bytes` starting at row0's
  // first element: whatever lies past `bytes` arrives as zeros.
  __device__ __forceinline__ void issue_bytes(const void* row0_base, uint32_t bytes, uint16_t* tile) const {
    const BufDesc d = buf_desc(row0_base, bytes);
    const uint32_t dst = lds_addr(tile) + (uint32_t)chunk0 * 16;
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) lds_dma16(d, dst + k * 64 * 16, voff[k]);
  }
  // Rows past valid_rows arrive as zeros.
  __device__ __forceinline__ void issue(const void* base, uint32_t stride_bytes, int row0, int valid_rows,
                                        uint16_t* tile) const {
    const int left = valid_rows - row0;
    const BufDesc d = buf_desc(reinterpret_cast<const char*>(base) + (size_t)row0 * stride_bytes,
                               left > 0 ? (uint32_t)left * stride_bytes : 0u);
    const uint32_t dst = lds_addr(tile) + (uint32_t)chunk0 * 16;
#pragma unroll
    for (int k = 0; k < PER_WAVE; ++k) lds_dma16(d, dst + k * 64 * 16, voff[k]);
  }
};

// Wave priority around MFMA-heavy sections: a wave issuing matrix work runs
// ahead of the co-resident wave, whose VALU work then fills the gaps.
#ifndef SDPA_PRIO
#define SDPA_PRIO 1
#endif
__device__ __forceinline__ void prio_mfma() {
  if constexpr (SDPA_PRIO) __builtin_amdgcn_s_setprio(1);
}
__device__ __forceinline__ void prio_valu() {
  if constexpr (SDPA_PRIO) __builtin_amdgcn_s_setprio(0);
}

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
