// Forward and backward attention for float32 inputs, computed in float32.
//
// Same definitions as the bf16 kernels (codelab "Speed up attention on GPU
// with cuDNN and TransformerEngine", "How attention works"; sink softmax of
// PR #2225), but every product and sum stays in fp32 (VALU FMA, no MFMA
// rounding of P or dS), so fp32 problems keep fp32 accuracy.  A workgroup of
// four waves owns a 64-row tile: each lane one query row (forward, dQ) or one
// key row (dK/dV), each wave a quarter of every 64-row tile on the other side
// (16 keys, or 16 query rows), staged in LDS and read as broadcasts.  The four
// waves' partial results are combined at the end in wave order (a fixed
// order, so results are reproducible).
//
// Attention dropout (dropout.h) draws one generator call per pair here: O
// accumulates kept probabilities only and is scaled by 1 / (1 - p) at the
// end; dV takes P * keep, dS = P (Z dP - delta) with Z = keep / (1 - p).
#include "dropout.h"
#include "launch.h"

namespace sdpa {

constexpr int kF32Tile = 64;
constexpr int kF32Waves = 4;
constexpr int kF32Part = kF32Tile / kF32Waves;  // rows of the other side per wave and tile

// Rows [r0, r0 + 64) of a [rows][D] fp32 tensor slice (rows `stride`
// floats apart) into an LDS tile, zeros past `valid`; all threads help.
template <int D>
__device__ __forceinline__ void load_tile_f32(float (*dst)[D], const float* src, size_t stride, int r0, int valid,
                                              int tid) {
  for (int idx = tid; idx < kF32Tile * D; idx += kF32Tile * kF32Waves) {
    const int r = idx / D, d = idx % D;
    dst[r][d] = r0 + r < valid ? src[(size_t)(r0 + r) * stride + d] : 0.0f;
  }
}

template <int DQK, int DV>
__global__ __launch_bounds__(256) void fwd_f32_kernel(KArgs a) {
  __shared__ float Ks[kF32Tile][DQK];
  __shared__ float Vs[kF32Tile][DV];
  __shared__ float part[kF32Waves - 1][kF32Tile][DV + 2];  // waves 1..3: o, m, l per row
  const int tid = threadIdx.x, w = wave_id(tid), lane = tid & 63;
  const int per = a.B * a.Hq;
  const int qt = a.n_tiles - 1 - blockIdx.x / per;
  const int b = (blockIdx.x % per) / a.Hq, h = (blockIdx.x % per) % a.Hq, g = h / a.G;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  const DropGen dg = drop_gen(a);
  const int i0 = qt * kF32Tile, qi = i0 + lane;
  const float* Q = static_cast<const float*>(a.q);

  float q[DQK], o[DV];
  for (int d = 0; d < DQK; ++d) q[d] = qi < m.L ? Q[((seq_row0(a, b) + qi) * a.Hq + h) * DQK + d] * a.scale : 0.0f;
  for (int d = 0; d < DV; ++d) o[d] = 0.0f;
  // The sink enters once: as wave 0's initial state.
  const bool sink = a.softmax_type != 0 && w == 0;
  float mrun = sink ? sink_logit(a, h) : -__builtin_inff();
  float l = sink ? 1.0f : 0.0f;

  int lo = 0, hi = -1;
  const int nrow = (i0 + kF32Tile < m.L ? i0 + kF32Tile : m.L) - 1;
  if (!key_range(m, i0, nrow, lo, hi)) { lo = 0; hi = -1; }
  const size_t kvrow = (size_t)a.Hkv;
  const float* Kb = static_cast<const float*>(a.k) + (seq_row0(a, b) * a.Hkv + g) * DQK;
  const float* Vb = static_cast<const float*>(a.v) + (seq_row0(a, b) * a.Hkv + g) * DV;
  for (int j0 = (lo / kF32Tile) * kF32Tile; hi >= 0 && j0 <= hi; j0 += kF32Tile) {
    __syncthreads();
    load_tile_f32<DQK>(Ks, Kb, kvrow * DQK, j0, m.L, tid);
    load_tile_f32<DV>(Vs, Vb, kvrow * DV, j0, m.L, tid);
    __syncthreads();
    for (int r = w * kF32Part; r < (w + 1) * kF32Part; ++r) {
      if (!visible(m, qi, j0 + r)) continue;
      float s = 0.0f;
      for (int d = 0; d < DQK; ++d) s = fmaf(q[d], Ks[r][d], s);
      const float kp = (dg.t > 0 && !drop_keep_pair(dg, b * a.Hq + h, qi, j0 + r)) ? 0.0f : 1.0f;
      if (s > mrun) {
        const float c = expf(mrun - s);
        l = l * c + 1.0f;
        for (int d = 0; d < DV; ++d) o[d] = fmaf(o[d], c, kp * Vs[r][d]);
        mrun = s;
      } else {
        const float p = expf(s - mrun);
        l += p;
        for (int d = 0; d < DV; ++d) o[d] = fmaf(kp * p, Vs[r][d], o[d]);
      }
    }
  }
  // Combine the waves' (m, l, o) in wave order.
  if (w > 0) {
    for (int d = 0; d < DV; ++d) part[w - 1][lane][d] = o[d];
    part[w - 1][lane][DV] = mrun;
    part[w - 1][lane][DV + 1] = l;
  }
  __syncthreads();
  if (w == 0) {
    for (int k = 0; k < kF32Waves - 1; ++k) {
      const float m2 = part[k][lane][DV], l2 = part[k][lane][DV + 1];
      const float mn = fmaxf(mrun, m2);
      if (mn == -__builtin_inff()) continue;  // both empty
      const float c1 = expf(mrun - mn), c2 = expf(m2 - mn);
      l = l * c1 + l2 * c2;
      for (int d = 0; d < DV; ++d) o[d] = o[d] * c1 + part[k][lane][d] * c2;
      mrun = mn;
    }
    if (qi < seq_rows(a, b)) {
      const float inv = l > 0.0f ? (dg.t > 0 ? dg.scale : 1.0f) / l : 0.0f;
      float* O = static_cast<float*>(a.out_o) + ((seq_row0(a, b) + qi) * a.Hq + h) * DV;
      for (int d = 0; d < DV; ++d) O[d] = o[d] * inv;
    }
    if (qi < a.S) {
      a.out_lse[((size_t)b * a.Hq + h) * a.S + qi] = l > 0.0f ? mrun + logf(l) : -__builtin_inff();
    }
  }
}

template <int DQK, int DV>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(KArgs a) {
  __shared__ float Qs[kF32Tile][DQK];
  __shared__ float dOs[kF32Tile][DV];
  __shared__ float lse_s[kF32Tile], delta_s[kF32Tile];
  __shared__ float part[kF32Waves - 1][kF32Tile][DQK + DV];  // waves 1..3: dk, dv per key
  const int tid = threadIdx.x, w = wave_id(tid), lane = tid & 63;
  const int per = a.B * a.Hkv;
  const int kt = blockIdx.x / per;
  const int b = (blockIdx.x % per) / a.Hkv, g = (blockIdx.x % per) % a.Hkv;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  const DropGen dg = drop_gen(a);
  const int j0 = kt * kF32Tile, kj = j0 + lane;
  float kk[DQK], vv[DV], dk[DQK], dv[DV];
  {
    const size_t row = (seq_row0(a, b) + kj) * a.Hkv + g;
    for (int d = 0; d < DQK; ++d) { kk[d] = kj < m.L ? static_cast<const float*>(a.k)[row * DQK + d] : 0.0f; dk[d] = 0.0f; }
    for (int d = 0; d < DV; ++d) { vv[d] = kj < m.L ? static_cast<const float*>(a.v)[row * DV + d] : 0.0f; dv[d] = 0.0f; }
  }
  int lo = 0, hi = -1;
  if (!query_range(m, j0, j0 + kF32Tile - 1, lo, hi)) { lo = 0; hi = -1; }
  const size_t qrow = (size_t)a.Hq;
  for (int hi_ = 0; hi_ < a.G; ++hi_) {
    const int h = g * a.G + hi_;
    const float* Qb = static_cast<const float*>(a.q) + (seq_row0(a, b) * a.Hq + h) * DQK;
    const float* dOb = static_cast<const float*>(a.d_o) + (seq_row0(a, b) * a.Hq + h) * DV;
    for (int q0 = (lo / kF32Tile) * kF32Tile; hi >= 0 && q0 <= hi; q0 += kF32Tile) {
      __syncthreads();
      load_tile_f32<DQK>(Qs, Qb, qrow * DQK, q0, m.L, tid);
      load_tile_f32<DV>(dOs, dOb, qrow * DV, q0, m.L, tid);
      if (w == 0) {
        const int i = q0 + lane;
        lse_s[lane] = i < m.L ? a.lse[((size_t)b * a.Hq + h) * a.S + i] : 0.0f;
        delta_s[lane] = i < m.L ? a.delta[((size_t)b * a.Hq + h) * a.S + i] : 0.0f;
      }
      __syncthreads();
      for (int r = w * kF32Part; r < (w + 1) * kF32Part; ++r) {
        if (!visible(m, q0 + r, kj)) continue;
        float s = 0.0f, dp = 0.0f;
        for (int d = 0; d < DQK; ++d) s = fmaf(Qs[r][d], kk[d], s);
        for (int d = 0; d < DV; ++d) dp = fmaf(dOs[r][d], vv[d], dp);
        const float p = expf(s * a.scale - lse_s[r]);
        float pk = p;
        if (dg.t > 0) {
          const bool kp = drop_keep_pair(dg, b * a.Hq + h, q0 + r, kj);
          pk = kp ? p : 0.0f;
          dp = kp ? dp * dg.scale : 0.0f;
        }
        const float ds = p * (dp - delta_s[r]);
        for (int d = 0; d < DV; ++d) dv[d] = fmaf(pk, dOs[r][d], dv[d]);
        for (int d = 0; d < DQK; ++d) dk[d] = fmaf(ds, Qs[r][d], dk[d]);
      }
    }
  }
  // Sum the waves' partials in wave order.
  if (w > 0) {
    for (int d = 0; d < DQK; ++d) part[w - 1][lane][d] = dk[d];
    for (int d = 0; d < DV; ++d) part[w - 1][lane][DQK + d] = dv[d];
  }
  __syncthreads();
  if (w == 0 && kj < seq_rows(a, b)) {
    for (int k = 0; k < kF32Waves - 1; ++k) {
      for (int d = 0; d < DQK; ++d) dk[d] += part[k][lane][d];
      for (int d = 0; d < DV; ++d) dv[d] += part[k][lane][DQK + d];
    }
    const size_t row = (seq_row0(a, b) + kj) * a.Hkv + g;
    for (int d = 0; d < DQK; ++d) static_cast<float*>(a.dk)[row * DQK + d] = dk[d] * a.scale;
    const float zs = dg.t > 0 ? dg.scale : 1.0f;
    for (int d = 0; d < DV; ++d) static_cast<float*>(a.dv)[row * DV + d] = dv[d] * zs;
  }
}

template <int DQK, int DV>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(KArgs a) {
  __shared__ float Ks[kF32Tile][DQK];
  __shared__ float Vs[kF32Tile][DV];
  __shared__ float part[kF32Waves - 1][kF32Tile][DQK];  // waves 1..3: dq per row
  const int tid = threadIdx.x, w = wave_id(tid), lane = tid & 63;
  const int per = a.B * a.Hq;
  const int qt = a.n_tiles - 1 - blockIdx.x / per;
  const int b = (blockIdx.x % per) / a.Hq, h = (blockIdx.x % per) % a.Hq, g = h / a.G;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  const DropGen dg = drop_gen(a);
  const int i0 = qt * kF32Tile, qi = i0 + lane;
  float q[DQK], dov[DV], dq[DQK];
  float lse = 0.0f, dl = 0.0f;
  {
    const size_t row = (seq_row0(a, b) + qi) * a.Hq + h;
    for (int d = 0; d < DQK; ++d) { q[d] = qi < m.L ? static_cast<const float*>(a.q)[row * DQK + d] : 0.0f; dq[d] = 0.0f; }
    for (int d = 0; d < DV; ++d) dov[d] = qi < m.L ? static_cast<const float*>(a.d_o)[row * DV + d] : 0.0f;
    if (qi < m.L) {
      lse = a.lse[((size_t)b * a.Hq + h) * a.S + qi];
      dl = a.delta[((size_t)b * a.Hq + h) * a.S + qi];
    }
  }
  int lo = 0, hi = -1;
  const int nrow = (i0 + kF32Tile < m.L ? i0 + kF32Tile : m.L) - 1;
  if (!key_range(m, i0, nrow, lo, hi)) { lo = 0; hi = -1; }
  const size_t kvrow = (size_t)a.Hkv;
  const float* Kb = static_cast<const float*>(a.k) + (seq_row0(a, b) * a.Hkv + g) * DQK;
  const float* Vb = static_cast<const float*>(a.v) + (seq_row0(a, b) * a.Hkv + g) * DV;
  for (int j0 = (lo / kF32Tile) * kF32Tile; hi >= 0 && j0 <= hi; j0 += kF32Tile) {
    __syncthreads();
    load_tile_f32<DQK>(Ks, Kb, kvrow * DQK, j0, m.L, tid);
    load_tile_f32<DV>(Vs, Vb, kvrow * DV, j0, m.L, tid);
    __syncthreads();
    for (int r = w * kF32Part; r < (w + 1) * kF32Part; ++r) {
      if (!visible(m, qi, j0 + r)) continue;
      float s = 0.0f, dp = 0.0f;
      for (int d = 0; d < DQK; ++d) s = fmaf(q[d], Ks[r][d], s);
      for (int d = 0; d < DV; ++d) dp = fmaf(dov[d], Vs[r][d], dp);
      const float p = expf(s * a.scale - lse);
      if (dg.t > 0) dp = drop_keep_pair(dg, b * a.Hq + h, qi, j0 + r) ? dp * dg.scale : 0.0f;
      const float ds = p * (dp - dl);
      for (int d = 0; d < DQK; ++d) dq[d] = fmaf(ds, Ks[r][d], dq[d]);
    }
  }
  if (w > 0)
    for (int d = 0; d < DQK; ++d) part[w - 1][lane][d] = dq[d];
  __syncthreads();
  if (w == 0 && qi < seq_rows(a, b)) {
    for (int k = 0; k < kF32Waves - 1; ++k)
      for (int d = 0; d < DQK; ++d) dq[d] += part[k][lane][d];
    float* dQ = static_cast<float*>(a.dq) + ((seq_row0(a, b) + qi) * a.Hq + h) * DQK;
    for (int d = 0; d < DQK; ++d) dQ[d] = dq[d] * a.scale;
  }
}

bool fwd_f32_tiles(int dqk, int dv, int* bm, int* bn) {
  if (dqk == 64 && dv == 64) { *bm = kF32Tile; *bn = kF32Tile; return true; }
  return false;
}

hipError_t launch_fwd_f32(const KArgs& a0, int dqk, int dv, hipStream_t stream) {
  if (!(dqk == 64 && dv == 64)) return hipErrorInvalidValue;
  KArgs a = a0;
  a.n_tiles = (a.S + kF32Tile - 1) / kF32Tile;
  hipLaunchKernelGGL((fwd_f32_kernel<64, 64>), dim3((unsigned)(a.n_tiles * a.B * a.Hq)), dim3(kF32Tile * kF32Waves), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_f32(const KArgs& a0, int dqk, int dv, hipStream_t stream) {
  if (!(dqk == 64 && dv == 64)) return hipErrorInvalidValue;
  KArgs a = a0;
  a.n_tiles = (a.S + kF32Tile - 1) / kF32Tile;
  hipLaunchKernelGGL((bwd_dkdv_f32_kernel<64, 64>), dim3((unsigned)(a.n_tiles * a.B * a.Hkv)), dim3(kF32Tile * kF32Waves), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_f32(const KArgs& a0, int dqk, int dv, hipStream_t stream) {
  if (!(dqk == 64 && dv == 64)) return hipErrorInvalidValue;
  KArgs a = a0;
  a.n_tiles = (a.S + kF32Tile - 1) / kF32Tile;
  hipLaunchKernelGGL((bwd_dq_f32_kernel<64, 64>), dim3((unsigned)(a.n_tiles * a.B * a.Hq)), dim3(kF32Tile * kF32Waves), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sdpa
