// FP8 attention backward: E4M3 Q, K, V and E5M2 dO with per-tensor descales,
// gfx950 MFMA 32x32x64 f8f6f4 (operand formats chosen per product), fp32
// softmax arithmetic, bf16 dQ, dK, dV.
//
// Computes (codelab "Speed up attention on GPU with cuDNN and
// TransformerEngine", section 10: FP8 autocast with the HYBRID recipe, E4M3
// forward tensors and E5M2 gradients; the arithmetic is this build's reading,
// stated in the header):
//     P_ij  = exp(scale dq dk (Q8_i . K8_j) - LSE_i)      (visible pairs)
//     delta_i = ddo (dO8_i . O_i),  dP_ij = ddo dv (dO8_i . V8_j)
//     dS_ij = P_ij (dP_ij - delta_i)
//     dV_j  = ddo / 256 sum_i E4M3(256 P_ij) dO8_i
//     dK_j  = scale dq / s_ds sum_i E5M2(s_ds dS_ij) Q8_i
//     dQ_i  = scale dk / s_ds sum_j E5M2(s_ds dS_ij) K8_j
// summed over the query heads of a KV head's group for dK, dV; amax = max |dS|.
//
// Launch order: transposes of K, Q and dO into the workspace ([dims]
// [positions] with the positions of each 64-group in the byte order of the
// accumulator-side operands, fp8_key_slot), then the dQ kernel, which also
// runs the pre-pass for its rows (delta, LSE log2 e, sink-gradient partials
// per 32 rows), and the dK/dV kernel; both recompute S and dP
// (deterministic, no atomics on the gradients).
//
// Products and operand formats (A x B, cbsz / blgp = 0 E4M3, 1 E5M2):
//   dQ kernel (lane = query row, 16 keys of each 32-key block per lane):
//     S^T  = K Q^T     A K rows (LDS)        B Q row (registers)   E4M3 x E4M3
//     dP^T = V dO^T    A V rows (LDS)        B dO row (registers)  E4M3 x E5M2
//     dQ^T += K^T dS8  A K^T rows (LDS)      B dS8 (accumulators)  E4M3 x E5M2
//   dK/dV kernel (lane = key, 16 rows of each 32-row block per lane):
//     S    = Q K^T     A Q rows (LDS)        B K row (registers)   E4M3 x E4M3
//     dP   = dO V^T    A dO rows (LDS)       B V row (registers)   E5M2 x E4M3
//     dV^T += dO^T P8  A dO^T rows (LDS)     B P8 (accumulators)   E5M2 x E4M3
//     dK^T += Q^T dS8  A Q^T rows (LDS)      B dS8 (accumulators)  E4M3 x E5M2
// The pre-pass stores the per-row terms already scaled for the element work:
// l8 = LSE log2 e - 8, so exp2(s c8 - l8) = 256 P is the E4M3 input, and
// delta' = delta s_ds / 256, so 256 P (dP' - delta') with dP' = dP s_ds / 256
// is s_ds dS, the E5M2 input: per element one FMA, one exp, one FMA, one
// multiply and one clamp, plus the mask where a step needs it.
// A 32x32x64 operand is 32 bytes per lane: row (or column) l % 32, half l / 32;
// an A lane and a B lane of the same half pair their bytes one to one.
// Row-major tiles are read as chunks 4k + hf and 4k + 2 + hf of a row for
// k-step k (both operands alike); the accumulator-side operand packs its 32
// elements of two 32-wide blocks in element order, matched by the permuted
// transposed tiles.
#include <type_traits>

#include "launch.h"

namespace sdpa {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kE4 = 0, kE5 = 1;

template <int FA, int FB>
__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, 0, 0, 0, 0);
}
__device__ __forceinline__ i32x8 cat16(const u32x4& lo, const u32x4& hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
__device__ __forceinline__ i32x8 words8(const uint32_t (&w)[8]) {
  return i32x8{(int)w[0], (int)w[1], (int)w[2], (int)w[3], (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
}
// E5M2 code -> float, exact: the code is the high byte of an IEEE half.
__device__ __forceinline__ float e5m2_value(uint32_t code) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)((code & 0xffu) << 8));
}
// Four values -> four codes in one word (element e in byte e), round to
// nearest even; E4M3 inputs here never exceed 256, E5M2 ones are clamped to
// the format's range first (the conversion alone turns overflow into NaN).
__device__ __forceinline__ uint32_t pack_e4m3(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, w, true);
  return (uint32_t)w;
}
__device__ __forceinline__ float clamp_e5m2(float x) { return __builtin_amdgcn_fmed3f(x, -57344.0f, 57344.0f); }
__device__ __forceinline__ uint32_t pack_e5m2(float x0, float x1, float x2, float x3) {
  int w = __builtin_amdgcn_cvt_pk_bf8_f32(clamp_e5m2(x0), clamp_e5m2(x1), 0, false);
  w = __builtin_amdgcn_cvt_pk_bf8_f32(clamp_e5m2(x2), clamp_e5m2(x3), w, true);
  return (uint32_t)w;
}
// Maximum over the workgroup's four waves, then one atomic max on the float
// bits (values are non-negative, so the unsigned order is the float order).
__device__ __forceinline__ void amax_atomic(float v, float* red4, float* out, int tid) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  if ((tid & 63) == 0) red4[tid >> 6] = v;
  __syncthreads();
  if (tid == 0) atomicMax(reinterpret_cast<unsigned int*>(out),
                          __float_as_uint(fmaxf(fmaxf(red4[0], red4[1]), fmaxf(red4[2], red4[3]))));
}

}  // namespace

__global__ void fp8_amax_zero_kernel(float* amax) {
  if (threadIdx.x == 0) amax[0] = 0.0f;
}

// codes [rows, heads, D] per batch -> [B, heads, D, s_pad] with the positions
// of each 64-group in fp8_key_slot order; positions at or past the batch's
// valid length are zero.  One workgroup per (batch, head, 64 positions): the
// 64 rows arrive in LDS with 16-byte loads (D / 16 consecutive threads per
// row), then each thread writes 16-byte pieces of the [D][64] output, slot
// t of a row holding position 32 (t / 16 % 2) + acc_row(t % 16, t / 32).
template <int D>
__global__ __launch_bounds__(256) void fp8_transpose_kernel(KArgs a, const uint8_t* src, int heads, uint8_t* dst) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[64 * D];
  const int groups = a.s_pad / 64;
  const int grp = blockIdx.x % groups;
  const int hh = (blockIdx.x / groups) % heads, b = blockIdx.x / (groups * heads);
  const int tid = threadIdx.x;
  const int L = seq_len(a, b), j0 = grp * 64;
#pragma unroll
  for (int c = tid; c < 64 * D / 16; c += 256) {
    const int row = c / (D / 16), ch = c % (D / 16);
    u32x4 v = {0u, 0u, 0u, 0u};
    if (j0 + row < L) v = *reinterpret_cast<const u32x4*>(src + ((seq_row0(a, b) + j0 + row) * heads + hh) * D + ch * 16);
    *reinterpret_cast<u32x4*>(tile + row * D + ch * 16) = v;
  }
  __syncthreads();
  uint8_t* out = dst + ((size_t)b * heads + hh) * D * a.s_pad + j0;
#pragma unroll
  for (int c = tid; c < D * 4; c += 256) {
    const int d = c / 4, t0 = (c % 4) * 16;  // dim row d, slots t0 .. t0+15
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t word = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = t0 + q * 4 + e;
        const int k = ((t >> 4) & 1) * 32 + acc_row(t & 15, t >> 5);
        word |= (uint32_t)tile[k * D + d] << (8 * e);
      }
      w[q] = word;
    }
    *reinterpret_cast<u32x4*>(out + (size_t)d * a.s_pad + t0) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

template <int D>
struct Fp8BwdCfg {
  static constexpr int BM = 128;  // dQ: query rows per workgroup (32 per wave)
  static constexpr int BN = 64;   // dQ: keys per step; dK/dV: query rows per step
  static constexpr int BK = 128;  // dK/dV: keys per workgroup (32 per wave)
  static constexpr int NT = 256;
  static constexpr int KCH = D / 16;  // 16-byte chunks of a D-byte row
  static constexpr int T = 64 * D;    // bytes of a [64][D] row tile or a [D][64] transposed tile
  static constexpr int NKS = D / 64;  // k-steps over the head dims
};

// ---- dQ ----------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_fp8_kernel(KArgs a) {
  using C = Fp8BwdCfg<D>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * 3 * C::T];
  __shared__ float red4[4];
  auto krows = [&](int buf) __attribute__((always_inline)) { return lds + buf * 3 * C::T; };
  auto vrows = [&](int buf) __attribute__((always_inline)) { return lds + buf * 3 * C::T + C::T; };
  auto kcols = [&](int buf) __attribute__((always_inline)) { return lds + buf * 3 * C::T + 2 * C::T; };

  const int tid = threadIdx.x, w = wave_id(tid), lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  // Same tile order as the forward: heavy query tiles first, the heads of a
  // GQA group on consecutive ids kept on one XCD.
  int b, h, qt;
  {
    const int N = a.B * a.Hq * a.n_tiles, chunk = a.G, full = (N / (8 * chunk)) * (8 * chunk);
    int l = blockIdx.x;
    if (l < full) {
      const int xcd = l & 7, slot = l >> 3;
      l = ((slot / chunk) * 8 + xcd) * chunk + slot % chunk;
    }
    const int per_tile = a.B * a.Hq;
    qt = a.n_tiles - 1 - l / per_tile;
    b = (l % per_tile) / a.Hq;
    h = (l % per_tile) % a.Hq;
  }
  const int g = h / a.G;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  const int i0 = qt * C::BM, qi = i0 + w * 32 + l32;
  int klo, khi;
  row_key_bounds(m, qi, klo, khi);

  // Q and dO rows of this lane's query (rows past the valid length read zeros).
  i32x8 qreg[C::NKS], oreg[C::NKS];
  {
    const size_t stride = (size_t)a.Hq * D;
    const __amdgpu_buffer_rsrc_t qres = buf_rsrc(static_cast<const uint8_t*>(a.q) + (seq_row0(a, b) * a.Hq + h) * D,
                                                 (uint32_t)(m.L * stride));
    const __amdgpu_buffer_rsrc_t ores = buf_rsrc(static_cast<const uint8_t*>(a.d_o) + (seq_row0(a, b) * a.Hq + h) * D,
                                                 (uint32_t)(m.L * stride));
#pragma unroll
    for (int k = 0; k < C::NKS; ++k) {
      qreg[k] = cat16(buf_load16(qres, (uint32_t)(qi * stride + (4 * k + hf) * 16)),
                      buf_load16(qres, (uint32_t)(qi * stride + (4 * k + 2 + hf) * 16)));
      oreg[k] = cat16(buf_load16(ores, (uint32_t)(qi * stride + (4 * k + hf) * 16)),
                      buf_load16(ores, (uint32_t)(qi * stride + (4 * k + 2 + hf) * 16)));
    }
  }
  // Backward pre-pass for this wave's 32 rows, fused here (the dK/dV kernel
  // runs after this one): delta = rowsum(dO * O) from the dequantized dO
  // codes (each lane half holds half of the row's dims), stored pre-scaled
  // as delta s_ds / 256 with LSE log2 e - 8 for both kernels (0 past the
  // valid length); for a sink logit z, the partial sum over the 32 rows of
  // dL/dz_i = -exp(z - LSE_i) delta_i, added up over the chunks later.
  float l8 = 0.0f, dl = 0.0f;  // LSE log2 e - 8, delta s_ds / 256
  {
    const size_t stride = (size_t)a.Hq * D;  // elements between rows
    const __amdgpu_buffer_rsrc_t outres = buf_rsrc(static_cast<const uint16_t*>(a.o) + (seq_row0(a, b) * a.Hq + h) * D,
                                                   (uint32_t)(m.L * stride * 2));
    float part = 0.0f;
#pragma unroll
    for (int k = 0; k < C::NKS; ++k)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int ch = 4 * k + 2 * c + hf;  // 16-dim chunk held in words 4c .. 4c+3 of oreg[k]
        const u32x4 o0 = buf_load16(outres, (uint32_t)((qi * stride + ch * 16) * 2));
        const u32x4 o1 = buf_load16(outres, (uint32_t)((qi * stride + ch * 16 + 8) * 2));
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t ow = e < 8 ? o0[e >> 1] : o1[(e - 8) >> 1];
          const float ov = (e & 1) ? bf16_hi(ow) : bf16_lo(ow);
          part += e5m2_value((uint32_t)oreg[k][4 * c + (e >> 2)] >> (8 * (e & 3))) * ov;
        }
      }
    const float delta = qi < m.L ? halves_sum(part) * a.fp8_descale[3] : 0.0f;
    const size_t row = ((size_t)b * a.Hq + h) * a.S + qi;
    const float lse = qi < m.L ? a.lse[row] : 0.0f;
    l8 = qi < m.L ? lse * kLog2e - 8.0f : 0.0f;
    dl = delta * (a.ds_scale[0] * (1.0f / 256.0f));
    if (hf == 0 && qi < a.S) {
      a.delta[row] = dl;
      a.lse2[row] = l8;
    }
    if (a.softmax_type != 0) {
      float dz = (hf == 0 && qi < m.L && lse > -__builtin_inff()) ? -expf(sink_logit(a, h) - lse) * delta : 0.0f;
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) dz += __shfl_xor(dz, off);
      const int qw0 = i0 + w * 32;
      if (lane == 0 && qw0 < a.S) a.dz_partial[((size_t)b * a.Hq + h) * a.n_chunks + qw0 / 32] = dz;
    }
  }
  const float dsk = a.fp8_descale[1];
  const float s_ds = a.ds_scale[0];
  const float c8 = a.scale_log2 * a.fp8_descale[0] * dsk;                      // raw score -> log2 units
  const float cdp = a.fp8_descale[3] * a.fp8_descale[2] * s_ds * (1.0f / 256.0f);  // raw dP -> dP s_ds / 256
  // The dQ products need only x = 256 P (cdp dP_raw - delta'), so cdp moves
  // into the exponent and delta' / cdp into the start of the dP accumulator:
  // x = exp2(s c8 - (l8 - log2 cdp)) (dP_raw - delta' / cdp), one multiply
  // per element (the descales and s_ds are positive).
  const float l8c = l8 - __log2f(cdp);
  f32x16 dinit;
#pragma unroll
  for (int i = 0; i < 16; ++i) dinit[i] = -dl / cdp;

  int lo = 0, hi = -1;
  const int nrow = (i0 + C::BM < m.L ? i0 + C::BM : m.L) - 1;
  if (!key_range(m, i0, nrow, lo, hi)) { lo = 0; hi = -1; }
  const int kt0 = lo / C::BN, kt1 = hi < 0 ? -1 : hi / C::BN;
  int fa = kt0, fb = kt0;  // tiles every row of the workgroup sees in full: [fa, fb)
  {
    int f0, f1;
    if (kt0 <= kt1 && full_key_tiles(m, i0, C::BM, C::BN, f0, f1)) {
      fa = f0 < kt0 ? kt0 : f0;
      fb = (f1 > kt1 ? kt1 : f1) + 1;
      if (fb < fa) fb = fa;
    }
  }

  const uint8_t* Kg = static_cast<const uint8_t*>(a.k) + (seq_row0(a, b) * a.Hkv + g) * D;
  const uint8_t* Vg = static_cast<const uint8_t*>(a.v) + (seq_row0(a, b) * a.Hkv + g) * D;
  const uint8_t* KTg = a.kt_t + ((size_t)b * a.Hkv + g) * D * a.s_pad;
  const uint32_t kvstride = (uint32_t)(a.Hkv * D);
  const TileCopy<C::BN, C::KCH, C::NT> rcopy(tid, kvstride);
  const TileCopy<D, 4, C::NT> tcopy(tid, (uint32_t)a.s_pad);
  const RowReads<C::KCH> rrd(lane);
  uint32_t toff[2];  // transposed rows: chunks 2 hf and 2 hf + 1 (the positions of this lane's half)
#pragma unroll
  for (int c = 0; c < 2; ++c) toff[c] = (uint32_t)swz_off<4>(l32, 2 * hf + c);
  auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
    const int j0 = kt * C::BN;
    rcopy.issue(Kg, kvstride, j0, m.L, reinterpret_cast<uint16_t*>(krows(buf)));
    rcopy.issue(Vg, kvstride, j0, m.L, reinterpret_cast<uint16_t*>(vrows(buf)));
    tcopy.issue_bytes(KTg + j0, (uint32_t)(D * a.s_pad - j0), reinterpret_cast<uint16_t*>(kcols(buf)));
  };

  f32x16 dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dq[db] = f32x16{};
  float amax = 0.0f;

  if (kt0 <= kt1) issue(kt0, 0);
  lds_dma_wait();
  __syncthreads();
  // One key tile; MASKED applies the per-element visibility (tiles outside
  // [fa, fb)), a separate instantiation so full tiles carry no mask work.
  auto step = [&](int kt, auto masked_c) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int buf = (kt - kt0) & 1;
    if (kt < kt1) issue(kt + 1, buf ^ 1);
    const uint16_t* Ks = reinterpret_cast<const uint16_t*>(krows(buf));
    const uint16_t* Vs = reinterpret_cast<const uint16_t*>(vrows(buf));
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = dinit;
    }
#pragma unroll
    for (int k = 0; k < C::NKS; ++k)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = mfma_f8<kE4, kE4>(cat16(rrd.read(Ks, kb * 32, 2 * k), rrd.read(Ks, kb * 32, 2 * k + 1)), qreg[k], s[kb]);
        dp[kb] = mfma_f8<kE4, kE5>(cat16(rrd.read(Vs, kb * 32, 2 * k), rrd.read(Vs, kb * 32, 2 * k + 1)), oreg[k], dp[kb]);
      }
    // Element i of block kb: key j0 + kb*32 + acc_row(i, hf), query qi;
    // x = 256 P (dP' - delta') = s_ds dS.
    const int j0 = kt * C::BN;
    const int lo_r = klo - (j0 + hf * 4), hi_r = khi - (j0 + hf * 4);
    uint32_t dw[8];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * q + e, off = kb * 32 + q * 8 + e;
          float pp = fast_exp2(fmaf(s[kb][i], c8, -l8c));
          if constexpr (MASKED) pp = (off >= lo_r && off <= hi_r) ? pp : 0.0f;
          x[e] = pp * dp[kb][i];
          amax = fmaxf(amax, fabsf(x[e]));
        }
        dw[kb * 4 + q] = pack_e5m2(x[0], x[1], x[2], x[3]);
      }
    const i32x8 dsb = words8(dw);
    const uint8_t* KTs = kcols(buf);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const char* row = reinterpret_cast<const char*>(KTs) + db * 32 * 64;
      dq[db] = mfma_f8<kE4, kE5>(cat16(*reinterpret_cast<const u32x4*>(row + toff[0]),
                                       *reinterpret_cast<const u32x4*>(row + toff[1])),
                                 dsb, dq[db]);
    }
    lds_dma_wait();
    __syncthreads();
  };
  for (int kt = kt0; kt < fa; ++kt) step(kt, std::true_type{});
  for (int kt = fa; kt < fb; ++kt) step(kt, std::false_type{});
  for (int kt = fb; kt <= kt1; ++kt) step(kt, std::true_type{});

  const float mul = a.scale * dsk / s_ds;
  if (qi < seq_rows(a, b)) {
    uint16_t* dqp = static_cast<uint16_t*>(a.dq) + ((seq_row0(a, b) + qi) * a.Hq + h) * D + hf * 4;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const u32x2 val = {pack_bf16(dq[db][ig * 4] * mul, dq[db][ig * 4 + 1] * mul),
                           pack_bf16(dq[db][ig * 4 + 2] * mul, dq[db][ig * 4 + 3] * mul)};
        *reinterpret_cast<u32x2*>(dqp + db * 32 + ig * 8) = val;
      }
  }
  amax_atomic(amax / s_ds, red4, a.amax_out, tid);
}

// ---- dK, dV ------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dkdv_fp8_kernel(KArgs a) {
  using C = Fp8BwdCfg<D>;
  // Stage (64 query rows of one head): Q rows, dO rows, Q^T, dO^T, lse2, delta.
  constexpr int STAGE = 4 * C::T + 2 * 64 * 4;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];
  auto qrows = [&](int buf) __attribute__((always_inline)) { return lds + buf * STAGE; };
  auto orows = [&](int buf) __attribute__((always_inline)) { return lds + buf * STAGE + C::T; };
  auto qcols = [&](int buf) __attribute__((always_inline)) { return lds + buf * STAGE + 2 * C::T; };
  auto ocols = [&](int buf) __attribute__((always_inline)) { return lds + buf * STAGE + 3 * C::T; };
  auto lse_s = [&](int buf) __attribute__((always_inline)) { return reinterpret_cast<float*>(lds + buf * STAGE + 4 * C::T); };
  auto del_s = [&](int buf) __attribute__((always_inline)) { return lse_s(buf) + 64; };

  const int tid = threadIdx.x, w = wave_id(tid), lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  // Workgroup id -> (key tile, batch, kv head): consecutive ids cover one key
  // tile, so a (batch, kv head) keeps to one XCD when B * Hkv is a multiple of 8.
  // Head split hs of n_splits covers query heads hs*Gs .. hs*Gs+Gs-1 of the
  // group (small grids: few KV heads or batches); each split then writes
  // fp32 partials that a second kernel adds in split order.
  const int nsp = a.n_splits, Gs = a.G / nsp;
  const int kt = blockIdx.x / (a.B * a.Hkv * nsp);
  int r0 = blockIdx.x % (a.B * a.Hkv * nsp);
  const int hs = r0 % nsp;
  r0 /= nsp;
  const int b = r0 / a.Hkv, g = r0 % a.Hkv;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  const int j0 = kt * C::BK, kj = j0 + w * 32 + l32;
  int qlo_k, qhi_k;  // rows that see this lane's key
  col_query_bounds(m, kj, qlo_k, qhi_k);

  // K and V rows of this lane's key (keys past the valid length read zeros).
  i32x8 kreg[C::NKS], vreg[C::NKS];
  {
    const size_t stride = (size_t)a.Hkv * D;
    const __amdgpu_buffer_rsrc_t kres = buf_rsrc(static_cast<const uint8_t*>(a.k) + (seq_row0(a, b) * a.Hkv + g) * D,
                                                 (uint32_t)(m.L * stride));
    const __amdgpu_buffer_rsrc_t vres = buf_rsrc(static_cast<const uint8_t*>(a.v) + (seq_row0(a, b) * a.Hkv + g) * D,
                                                 (uint32_t)(m.L * stride));
#pragma unroll
    for (int k = 0; k < C::NKS; ++k) {
      kreg[k] = cat16(buf_load16(kres, (uint32_t)(kj * stride + (4 * k + hf) * 16)),
                      buf_load16(kres, (uint32_t)(kj * stride + (4 * k + 2 + hf) * 16)));
      vreg[k] = cat16(buf_load16(vres, (uint32_t)(kj * stride + (4 * k + hf) * 16)),
                      buf_load16(vres, (uint32_t)(kj * stride + (4 * k + 2 + hf) * 16)));
    }
  }
  const float dsq = a.fp8_descale[0], dso = a.fp8_descale[3];
  const float s_ds = a.ds_scale[0];
  const float c8 = a.scale_log2 * dsq * a.fp8_descale[1];
  const float cdp = dso * a.fp8_descale[2] * s_ds * (1.0f / 256.0f);
  // Rows that see all 32 keys of this wave (none if it holds keys past the
  // valid length): steps inside them need no mask.
  int all_lo, all_hi;
  {
    const int kw0 = j0 + w * 32;
    int lo_a, hi_a, lo_b, hi_b;
    col_query_bounds(m, kw0 + 31, lo_a, hi_a);
    col_query_bounds(m, kw0, lo_b, hi_b);
    all_lo = lo_a;
    all_hi = hi_b;
    if (kw0 + 31 >= m.L) {
      all_lo = 1;
      all_hi = 0;
    }
  }

  // Steps: (head of the group, 64-row block) pairs, heads outer, rows ascending.
  int qlo = 0, qhi = -1;
  if (!query_range(m, j0, j0 + C::BK - 1, qlo, qhi)) { qlo = 0; qhi = -1; }
  const int q_first = (qlo / 64) * 64;
  const int nsteps = qhi < 0 ? 0 : qhi / 64 - qlo / 64 + 1;
  const int T = nsteps * Gs;

  const size_t stride = (size_t)a.Hq * D;
  const TileCopy<64, C::KCH, C::NT> rcopy(tid, (uint32_t)stride);
  const TileCopy<D, 4, C::NT> tcopy(tid, (uint32_t)a.s_pad);
  const RowReads<C::KCH> rrd(lane);
  uint32_t toff[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) toff[c] = (uint32_t)swz_off<4>(l32, 2 * hf + c);
  auto issue = [&](int t, int buf) __attribute__((always_inline)) {
    const int hh = t / nsteps, q0 = q_first + (t - hh * nsteps) * 64;
    const int h = g * a.G + hs * Gs + hh;
    const uint8_t* Qg = static_cast<const uint8_t*>(a.q) + (seq_row0(a, b) * a.Hq + h) * D;
    const uint8_t* Og = static_cast<const uint8_t*>(a.d_o) + (seq_row0(a, b) * a.Hq + h) * D;
    rcopy.issue(Qg, (uint32_t)stride, q0, m.L, reinterpret_cast<uint16_t*>(qrows(buf)));
    rcopy.issue(Og, (uint32_t)stride, q0, m.L, reinterpret_cast<uint16_t*>(orows(buf)));
    const size_t tbase = ((size_t)b * a.Hq + h) * D * a.s_pad + q0;
    const uint32_t left = (uint32_t)(D * a.s_pad - q0);
    tcopy.issue_bytes(a.qt_t + tbase, left, reinterpret_cast<uint16_t*>(qcols(buf)));
    tcopy.issue_bytes(a.dot_t + tbase, left, reinterpret_cast<uint16_t*>(ocols(buf)));
    // lse2 (wave 0) and delta (wave 1) of rows q0 .. q0+63; rows past S read zeros.
    if (w < 2) {
      const float* src = (w == 0 ? a.lse2 : a.delta) + ((size_t)b * a.Hq + h) * a.S;
      lds_dma4(buf_desc(src, (uint32_t)a.S * 4), lds_addr(w == 0 ? lse_s(buf) : del_s(buf)), (uint32_t)(q0 + lane) * 4);
    }
  };

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  if (T > 0) issue(0, 0);
  lds_dma_wait();
  __syncthreads();
  // Step t = (head hh, rows q0 .. q0+63).  Steps whose 64 rows all see this
  // wave's 32 keys run without the mask: per head, steps [m0, m1) (per wave;
  // every wave still passes one barrier per step, in step order).
  auto step = [&](int t, int hh, int q0, auto masked_c) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked_c)::value;
    const int buf = t & 1;
    if (t + 1 < T) issue(t + 1, buf ^ 1);
    const uint16_t* Qs = reinterpret_cast<const uint16_t*>(qrows(buf));
    const uint16_t* Os = reinterpret_cast<const uint16_t*>(orows(buf));
    f32x16 s[2], dp[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      s[rb] = f32x16{};
      dp[rb] = f32x16{};
    }
#pragma unroll
    for (int k = 0; k < C::NKS; ++k)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        s[rb] = mfma_f8<kE4, kE4>(cat16(rrd.read(Qs, rb * 32, 2 * k), rrd.read(Qs, rb * 32, 2 * k + 1)), kreg[k], s[rb]);
        dp[rb] = mfma_f8<kE5, kE4>(cat16(rrd.read(Os, rb * 32, 2 * k), rrd.read(Os, rb * 32, 2 * k + 1)), vreg[k], dp[rb]);
      }
    // Element i of block rb: row q0 + rb*32 + acc_row(i, hf), key kj; its
    // P8 / dS8 byte is 16 rb + i (word 4 rb + i/4), the order of the
    // transposed tiles' slots.
    const float* ls = lse_s(buf);
    const float* dl = del_s(buf);
    const int lo_r = qlo_k - (q0 + hf * 4), hi_r = qhi_k - (q0 + hf * 4);
    uint32_t pw[8], dw[8];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ro = rb * 32 + q * 8 + hf * 4;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + ro);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(dl + ro);
        float pp[4], xx[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * q + e, off = rb * 32 + q * 8 + e;
          pp[e] = fast_exp2(fmaf(s[rb][i], c8, -l4[e]));  // 256 P
          if constexpr (MASKED) pp[e] = (off >= lo_r && off <= hi_r) ? pp[e] : 0.0f;
          xx[e] = pp[e] * fmaf(dp[rb][i], cdp, -d4[e]);    // s_ds dS
        }
        pw[rb * 4 + q] = pack_e4m3(pp[0], pp[1], pp[2], pp[3]);
        dw[rb * 4 + q] = pack_e5m2(xx[0], xx[1], xx[2], xx[3]);
      }
    const i32x8 pb = words8(pw), db8 = words8(dw);
    const uint8_t* QTs = qcols(buf);
    const uint8_t* OTs = ocols(buf);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const char* orow = reinterpret_cast<const char*>(OTs) + db * 32 * 64;
      const char* qrow = reinterpret_cast<const char*>(QTs) + db * 32 * 64;
      dv[db] = mfma_f8<kE5, kE4>(cat16(*reinterpret_cast<const u32x4*>(orow + toff[0]),
                                       *reinterpret_cast<const u32x4*>(orow + toff[1])),
                                 pb, dv[db]);
      dk[db] = mfma_f8<kE4, kE5>(cat16(*reinterpret_cast<const u32x4*>(qrow + toff[0]),
                                       *reinterpret_cast<const u32x4*>(qrow + toff[1])),
                                 db8, dk[db]);
    }
    lds_dma_wait();
    __syncthreads();
  };
  int m0 = nsteps, m1 = nsteps;
  if (all_lo <= all_hi) {
    m0 = all_lo <= q_first ? 0 : (all_lo - q_first + 63) / 64;
    const int last = all_hi - 63 - q_first;  // q0 + 63 <= all_hi  <=>  s <= last / 64
    m1 = last < 0 ? 0 : last / 64 + 1;
    m0 = m0 < nsteps ? m0 : nsteps;
    m1 = m1 < m0 ? m0 : (m1 < nsteps ? m1 : nsteps);
  }
  for (int hh = 0, t = 0; hh < Gs; ++hh) {
    for (int st = 0; st < m0; ++st, ++t) step(t, hh, q_first + st * 64, std::true_type{});
    for (int st = m0; st < m1; ++st, ++t) step(t, hh, q_first + st * 64, std::false_type{});
    for (int st = m1; st < nsteps; ++st, ++t) step(t, hh, q_first + st * 64, std::true_type{});
  }

  // Epilogue: lane owns key kj, dims db*32 + acc_row(i, hf).
  const float mk = a.scale * dsq / s_ds, mv = dso / 256.0f;
  if (nsp > 1) {
    // fp32 partials of this split, already scaled, in the padded layout
    // (row (hs*B + b)*S + kj of [.., Hkv, D]) the split-reduce kernel reads
    if (kj < seq_rows(a, b)) {
      const size_t row = ((size_t)(hs * a.B + b) * a.S + kj) * a.Hkv + g;
      float* dkp = a.kv_part + row * D + hf * 4;
      float* dvp = a.kv_part + (size_t)nsp * a.B * a.S * a.Hkv * D + row * D + hf * 4;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          *reinterpret_cast<f32x4*>(dkp + db * 32 + ig * 8) =
              f32x4{dk[db][ig * 4] * mk, dk[db][ig * 4 + 1] * mk, dk[db][ig * 4 + 2] * mk, dk[db][ig * 4 + 3] * mk};
          *reinterpret_cast<f32x4*>(dvp + db * 32 + ig * 8) =
              f32x4{dv[db][ig * 4] * mv, dv[db][ig * 4 + 1] * mv, dv[db][ig * 4 + 2] * mv, dv[db][ig * 4 + 3] * mv};
        }
    }
  } else if (kj < seq_rows(a, b)) {
    uint16_t* dkp = static_cast<uint16_t*>(a.dk) + ((seq_row0(a, b) + kj) * a.Hkv + g) * D + hf * 4;
    uint16_t* dvp = static_cast<uint16_t*>(a.dv) + ((seq_row0(a, b) + kj) * a.Hkv + g) * D + hf * 4;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        *reinterpret_cast<u32x2*>(dkp + db * 32 + ig * 8) =
            u32x2{pack_bf16(dk[db][ig * 4] * mk, dk[db][ig * 4 + 1] * mk),
                  pack_bf16(dk[db][ig * 4 + 2] * mk, dk[db][ig * 4 + 3] * mk)};
        *reinterpret_cast<u32x2*>(dvp + db * 32 + ig * 8) =
            u32x2{pack_bf16(dv[db][ig * 4] * mv, dv[db][ig * 4 + 1] * mv),
                  pack_bf16(dv[db][ig * 4 + 2] * mv, dv[db][ig * 4 + 3] * mv)};
      }
  }
}

template __global__ void fp8_transpose_kernel<64>(KArgs, const uint8_t*, int, uint8_t*);
template __global__ void fp8_transpose_kernel<128>(KArgs, const uint8_t*, int, uint8_t*);
template __global__ void bwd_dq_fp8_kernel<64>(KArgs);
template __global__ void bwd_dq_fp8_kernel<128>(KArgs);
template __global__ void bwd_dkdv_fp8_kernel<64>(KArgs);
template __global__ void bwd_dkdv_fp8_kernel<128>(KArgs);

size_t fp8_bwd_transposed_bytes(int B, int S, int Hq, int Hkv, int d) {
  const size_t s_pad = (size_t)((S + 63) / 64) * 64;
  return (size_t)B * d * s_pad * (size_t)(Hkv + 2 * Hq);
}

hipError_t launch_fp8_transpose(const KArgs& a, const void* src, int heads, uint8_t* dst, int d, hipStream_t stream) {
  const dim3 grid((unsigned)((long long)a.B * heads * (a.s_pad / 64)));
  if (d == 64) hipLaunchKernelGGL(fp8_transpose_kernel<64>, grid, dim3(256), 0, stream, a, static_cast<const uint8_t*>(src),
                                  heads, dst);
  else if (d == 128) hipLaunchKernelGGL(fp8_transpose_kernel<128>, grid, dim3(256), 0, stream, a,
                                        static_cast<const uint8_t*>(src), heads, dst);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_fp8_cfg(KArgs a, hipStream_t stream) {
  using C = Fp8BwdCfg<D>;
  a.s_pad = (a.S + 63) / 64 * 64;
  a.n_chunks = (a.S + 31) / 32;
  hipLaunchKernelGGL(fp8_amax_zero_kernel, dim3(1), dim3(64), 0, stream, a.amax_out);
  hipError_t e = launch_fp8_transpose(a, a.k, a.Hkv, a.kt_t, D, stream);
  if (e == hipSuccess) e = launch_fp8_transpose(a, a.q, a.Hq, a.qt_t, D, stream);
  if (e == hipSuccess) e = launch_fp8_transpose(a, a.d_o, a.Hq, a.dot_t, D, stream);
  if (e != hipSuccess) return e;
  a.n_tiles = (a.S + C::BM - 1) / C::BM;
  hipLaunchKernelGGL(bwd_dq_fp8_kernel<D>, dim3((unsigned)((long long)a.B * a.Hq * a.n_tiles)), dim3(C::NT), 0,
                     stream, a);
  const int nkt = (a.S + C::BK - 1) / C::BK;
  hipLaunchKernelGGL(bwd_dkdv_fp8_kernel<D>, dim3((unsigned)((long long)nkt * a.B * a.Hkv * a.n_splits)), dim3(C::NT),
                     0, stream, a);
  if (a.n_splits > 1) {
    // the partials are scaled already: add them with multiplier 1
    KArgs r = a;
    r.scale = 1.0f;
    r.drop_t = 0;
    e = launch_dkdv_split_reduce(r, D, D, stream);
    if (e != hipSuccess) return e;
  }
  if (a.d_offset && a.softmax_type != 0) return launch_dz_reduce(a, stream);
  return hipGetLastError();
}

hipError_t launch_bwd_fp8(const KArgs& a, int dqk, int dv, hipStream_t stream) {
  if (dqk == 64 && dv == 64) return launch_bwd_fp8_cfg<64>(a, stream);
  if (dqk == 128 && dv == 128) return launch_bwd_fp8_cfg<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace sdpa
