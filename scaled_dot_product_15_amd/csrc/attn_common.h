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
  float* delta;       // workspace [B,Hq,S]
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

}  // namespace sdpa
