// Forward and backward attention for float32 inputs, computed in float32.
//
// Same definitions as the bf16 kernels (codelab "Speed up attention on GPU
// with cuDNN and TransformerEngine", "How attention works"; sink softmax of
// PR #2225), but every product and sum stays in fp32 (VALU FMA, no MFMA
// rounding of P or dS), so fp32 problems keep fp32 accuracy.  One thread owns
// one query row (forward, dQ) or one key row (dK/dV); key/query tiles of 64
// rows are staged in LDS and read by all threads as broadcasts.
#include "launch.h"

namespace sdpa {

constexpr int kF32Tile = 64;

template <int DQK, int DV>
__global__ __launch_bounds__(64) void fwd_f32_kernel(KArgs a) {
  __shared__ float Ks[kF32Tile][DQK];
  __shared__ float Vs[kF32Tile][DV];
  const int tid = threadIdx.x;
  const int per = a.B * a.Hq;
  const int qt = a.n_tiles - 1 - blockIdx.x / per;
  const int b = (blockIdx.x % per) / a.Hq, h = (blockIdx.x % per) % a.Hq, g = h / a.G;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  const int i0 = qt * kF32Tile, qi = i0 + tid;
  const float* Q = static_cast<const float*>(a.q);
  const float* K = static_cast<const float*>(a.k);
  const float* V = static_cast<const float*>(a.v);

  float q[DQK], o[DV];
  for (int d = 0; d < DQK; ++d) q[d] = qi < m.L ? Q[((size_t)(b * a.S + qi) * a.Hq + h) * DQK + d] * a.scale : 0.0f;
  for (int d = 0; d < DV; ++d) o[d] = 0.0f;
  const bool sink = a.softmax_type != 0;
  float mrun = sink ? sink_logit(a, h) : -__builtin_inff();
  float l = sink ? 1.0f : 0.0f;

  int lo = 0, hi = -1;
  const int nrow = (i0 + kF32Tile < m.L ? i0 + kF32Tile : m.L) - 1;
  if (!key_range(m, i0, nrow, lo, hi)) { lo = 0; hi = -1; }
  for (int j0 = (lo / kF32Tile) * kF32Tile; hi >= 0 && j0 <= hi; j0 += kF32Tile) {
    __syncthreads();
    for (int r = 0; r < kF32Tile; ++r) {
      const int j = j0 + r;
      const size_t row = (size_t)(b * a.S + j) * a.Hkv + g;
      for (int d = tid; d < DQK; d += 64) Ks[r][d] = j < m.L ? K[row * DQK + d] : 0.0f;
      for (int d = tid; d < DV; d += 64) Vs[r][d] = j < m.L ? V[row * DV + d] : 0.0f;
    }
    __syncthreads();
    for (int r = 0; r < kF32Tile; ++r) {
      if (!visible(m, qi, j0 + r)) continue;
      float s = 0.0f;
      for (int d = 0; d < DQK; ++d) s = fmaf(q[d], Ks[r][d], s);
      if (s > mrun) {
        const float c = expf(mrun - s);
        l = l * c + 1.0f;
        for (int d = 0; d < DV; ++d) o[d] = fmaf(o[d], c, Vs[r][d]);
        mrun = s;
      } else {
        const float p = expf(s - mrun);
        l += p;
        for (int d = 0; d < DV; ++d) o[d] = fmaf(p, Vs[r][d], o[d]);
      }
    }
  }
  if (qi < a.S) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* O = static_cast<float*>(a.out_o) + ((size_t)(b * a.S + qi) * a.Hq + h) * DV;
    for (int d = 0; d < DV; ++d) O[d] = o[d] * inv;
    a.out_lse[((size_t)b * a.Hq + h) * a.S + qi] = l > 0.0f ? mrun + logf(l) : -__builtin_inff();
  }
}

template <int DQK, int DV>
__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(KArgs a) {
  __shared__ float Qs[kF32Tile][DQK];
  __shared__ float dOs[kF32Tile][DV];
  __shared__ float lse_s[kF32Tile], delta_s[kF32Tile];
  const int tid = threadIdx.x;
  const int per = a.B * a.Hkv;
  const int kt = blockIdx.x / per;
  const int b = (blockIdx.x % per) / a.Hkv, g = (blockIdx.x % per) % a.Hkv;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  const int j0 = kt * kF32Tile, kj = j0 + tid;
  const float* Q = static_cast<const float*>(a.q);
  const float* dO = static_cast<const float*>(a.d_o);
  float kk[DQK], vv[DV], dk[DQK], dv[DV];
  {
    const size_t row = (size_t)(b * a.S + kj) * a.Hkv + g;
    for (int d = 0; d < DQK; ++d) { kk[d] = kj < m.L ? static_cast<const float*>(a.k)[row * DQK + d] : 0.0f; dk[d] = 0.0f; }
    for (int d = 0; d < DV; ++d) { vv[d] = kj < m.L ? static_cast<const float*>(a.v)[row * DV + d] : 0.0f; dv[d] = 0.0f; }
  }
  int lo = 0, hi = -1;
  if (!query_range(m, j0, j0 + kF32Tile - 1, lo, hi)) { lo = 0; hi = -1; }
  for (int hi_ = 0; hi_ < a.G; ++hi_) {
    const int h = g * a.G + hi_;
    for (int q0 = (lo / kF32Tile) * kF32Tile; hi >= 0 && q0 <= hi; q0 += kF32Tile) {
      __syncthreads();
      for (int r = 0; r < kF32Tile; ++r) {
        const int i = q0 + r;
        const size_t row = (size_t)(b * a.S + i) * a.Hq + h;
        for (int d = tid; d < DQK; d += 64) Qs[r][d] = i < m.L ? Q[row * DQK + d] : 0.0f;
        for (int d = tid; d < DV; d += 64) dOs[r][d] = i < m.L ? dO[row * DV + d] : 0.0f;
      }
      {
        const int i = q0 + tid;
        lse_s[tid] = i < m.L ? a.lse[((size_t)b * a.Hq + h) * a.S + i] : 0.0f;
        delta_s[tid] = i < m.L ? a.delta[((size_t)b * a.Hq + h) * a.S + i] : 0.0f;
      }
      __syncthreads();
      for (int r = 0; r < kF32Tile; ++r) {
        if (!visible(m, q0 + r, kj)) continue;
        float s = 0.0f, dp = 0.0f;
        for (int d = 0; d < DQK; ++d) s = fmaf(Qs[r][d], kk[d], s);
        for (int d = 0; d < DV; ++d) dp = fmaf(dOs[r][d], vv[d], dp);
        const float p = expf(s * a.scale - lse_s[r]);
        const float ds = p * (dp - delta_s[r]);
        for (int d = 0; d < DV; ++d) dv[d] = fmaf(p, dOs[r][d], dv[d]);
        for (int d = 0; d < DQK; ++d) dk[d] = fmaf(ds, Qs[r][d], dk[d]);
      }
    }
  }
  if (kj < a.S) {
    const size_t row = (size_t)(b * a.S + kj) * a.Hkv + g;
    for (int d = 0; d < DQK; ++d) static_cast<float*>(a.dk)[row * DQK + d] = dk[d] * a.scale;
    for (int d = 0; d < DV; ++d) static_cast<float*>(a.dv)[row * DV + d] = dv[d];
  }
}

template <int DQK, int DV>
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(KArgs a) {
  __shared__ float Ks[kF32Tile][DQK];
  __shared__ float Vs[kF32Tile][DV];
  const int tid = threadIdx.x;
  const int per = a.B * a.Hq;
  const int qt = a.n_tiles - 1 - blockIdx.x / per;
  const int b = (blockIdx.x % per) / a.Hq, h = (blockIdx.x % per) % a.Hq, g = h / a.G;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  const int i0 = qt * kF32Tile, qi = i0 + tid;
  float q[DQK], dov[DV], dq[DQK];
  float lse = 0.0f, dl = 0.0f;
  {
    const size_t row = (size_t)(b * a.S + qi) * a.Hq + h;
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
  const float* K = static_cast<const float*>(a.k);
  const float* V = static_cast<const float*>(a.v);
  for (int j0 = (lo / kF32Tile) * kF32Tile; hi >= 0 && j0 <= hi; j0 += kF32Tile) {
    __syncthreads();
    for (int r = 0; r < kF32Tile; ++r) {
      const int j = j0 + r;
      const size_t row = (size_t)(b * a.S + j) * a.Hkv + g;
      for (int d = tid; d < DQK; d += 64) Ks[r][d] = j < m.L ? K[row * DQK + d] : 0.0f;
      for (int d = tid; d < DV; d += 64) Vs[r][d] = j < m.L ? V[row * DV + d] : 0.0f;
    }
    __syncthreads();
    for (int r = 0; r < kF32Tile; ++r) {
      if (!visible(m, qi, j0 + r)) continue;
      float s = 0.0f, dp = 0.0f;
      for (int d = 0; d < DQK; ++d) s = fmaf(q[d], Ks[r][d], s);
      for (int d = 0; d < DV; ++d) dp = fmaf(dov[d], Vs[r][d], dp);
      const float p = expf(s * a.scale - lse);
      const float ds = p * (dp - dl);
      for (int d = 0; d < DQK; ++d) dq[d] = fmaf(ds, Ks[r][d], dq[d]);
    }
  }
  if (qi < a.S) {
    float* dQ = static_cast<float*>(a.dq) + ((size_t)(b * a.S + qi) * a.Hq + h) * DQK;
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
  hipLaunchKernelGGL((fwd_f32_kernel<64, 64>), dim3((unsigned)(a.n_tiles * a.B * a.Hq)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_f32(const KArgs& a0, int dqk, int dv, hipStream_t stream) {
  if (!(dqk == 64 && dv == 64)) return hipErrorInvalidValue;
  KArgs a = a0;
  a.n_tiles = (a.S + kF32Tile - 1) / kF32Tile;
  hipLaunchKernelGGL((bwd_dkdv_f32_kernel<64, 64>), dim3((unsigned)(a.n_tiles * a.B * a.Hkv)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_f32(const KArgs& a0, int dqk, int dv, hipStream_t stream) {
  if (!(dqk == 64 && dv == 64)) return hipErrorInvalidValue;
  KArgs a = a0;
  a.n_tiles = (a.S + kF32Tile - 1) / kF32Tile;
  hipLaunchKernelGGL((bwd_dq_f32_kernel<64, 64>), dim3((unsigned)(a.n_tiles * a.B * a.Hq)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sdpa
