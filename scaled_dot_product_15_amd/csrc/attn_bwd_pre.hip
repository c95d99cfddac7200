// Backward pre-pass and the sink-gradient reduction.
//
// delta_i = sum_e dO_ie O_ie equals sum_j P_ij dP_ij, the term the softmax
// backward subtracts from dP; the pass also stores LSE_i * log2(e) for the
// base-2 recomputation of P in the backward kernels (PR #2225: the backward takes dz = dO and returns
// grad_q/k/v/softmax_offset).  For a sink logit z the gradient is
// dL/dz = -sum_i exp(z - LSE_i) delta_i: the sink enters only the softmax
// denominator and carries a zero value row.  Each block writes the partial
// sum of its rows; dz_reduce adds the partials of a head in a fixed order, so
// the result is bitwise reproducible.
#include "launch.h"

namespace sdpa {

template <typename T, int DV>
__global__ __launch_bounds__(256) void bwd_pre_kernel(KArgs a) {
  constexpr int EPC = 16 / sizeof(T);    // elements per 16-byte chunk
  constexpr int TPR = DV / EPC;          // threads per row
  constexpr int RPP = 256 / TPR;         // rows per pass
  static_assert(DV % EPC == 0 && 256 % TPR == 0 && kPreRows % RPP == 0, "row split");
  __shared__ float dzs[kPreRows];
  const int b = blockIdx.z, h = blockIdx.y, chunk = blockIdx.x;
  const int tid = threadIdx.x, rr = tid / TPR, part = tid % TPR;
  const int L = seq_len(a, b);
  const bool sink = a.softmax_type != 0;
  const float z = sink_logit(a, h);
  const T* O = static_cast<const T*>(a.o);
  const T* dO = static_cast<const T*>(a.d_o);
  for (int r0 = 0; r0 < kPreRows; r0 += RPP) {
    const int i = chunk * kPreRows + r0 + rr;
    float acc = 0.0f;
    if (i < L) {
      const size_t off = ((seq_row0(a, b) + i) * a.Hq + h) * DV + part * EPC;
      const u32x4 ov = ldg16(O + off), dv = ldg16(dO + off);
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc += __uint_as_float(ov[e] << 16) * __uint_as_float(dv[e] << 16);
          acc += __uint_as_float(ov[e] & 0xffff0000u) * __uint_as_float(dv[e] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) acc += __uint_as_float(ov[e]) * __uint_as_float(dv[e]);
      }
    }
#pragma unroll
    for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (part == 0) {
      if (i < a.S) {
        a.delta[((size_t)b * a.Hq + h) * a.S + i] = acc;
        a.lse2[((size_t)b * a.Hq + h) * a.S + i] = i < L ? a.lse[((size_t)b * a.Hq + h) * a.S + i] * kLog2e : 0.0f;
      }
      float dz = 0.0f;
      if (sink && i < L) dz = -expf(z - a.lse[((size_t)b * a.Hq + h) * a.S + i]) * acc;
      dzs[r0 + rr] = dz;
    }
  }
  if (sink) {
    __syncthreads();
    if (tid == 0) {
      float s = 0.0f;
      for (int r = 0; r < kPreRows; ++r) s += dzs[r];
      a.dz_partial[((size_t)b * a.Hq + h) * a.n_chunks + chunk] = s;
    }
  }
}

// d_offset[h] = sum of head h's B * n_chunks partials, one workgroup per
// head, in a fixed order: thread t adds partials t, t + 256, ... of the
// batch-major sequence (consecutive threads read consecutive chunks), then
// the 256 thread sums meet in a fixed pairwise tree.
constexpr int kDzThreads = 256;
__global__ __launch_bounds__(kDzThreads) void dz_reduce_kernel(KArgs a) {
  __shared__ float red[kDzThreads];
  const int h = blockIdx.x, t = threadIdx.x;
  const int n = a.B * a.n_chunks;
  float s = 0.0f;
  for (int i = t; i < n; i += kDzThreads) {
    const int b = i / a.n_chunks, c = i - b * a.n_chunks;
    s += a.dz_partial[((size_t)b * a.Hq + h) * a.n_chunks + c];
  }
  red[t] = s;
  __syncthreads();
  for (int w = kDzThreads / 2; w > 0; w >>= 1) {
    if (t < w) red[t] += red[t + w];
    __syncthreads();
  }
  if (t == 0) a.d_offset[h] = red[0];
}

hipError_t launch_bwd_pre(const KArgs& a, int dtype, int dv, hipStream_t stream) {
  const dim3 grid(a.n_chunks, a.Hq, a.B);
  if (dtype == 1 && dv == 64) hipLaunchKernelGGL((bwd_pre_kernel<uint16_t, 64>), grid, dim3(256), 0, stream, a);
  else if (dtype == 1 && dv == 128) hipLaunchKernelGGL((bwd_pre_kernel<uint16_t, 128>), grid, dim3(256), 0, stream, a);
  else if (dtype == 0 && dv == 64) hipLaunchKernelGGL((bwd_pre_kernel<float, 64>), grid, dim3(256), 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_dz_reduce(const KArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(dz_reduce_kernel, dim3(a.Hq), dim3(kDzThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sdpa
