// FP8 per-tensor scaling: quantization with amax, and the delayed-scaling
// scale update (codelab "Speed up attention on GPU with cuDNN and
// TransformerEngine", section 10: DelayedScaling with an amax history and the
// "max" rule; formats E4M3 / E5M2 of the OCP 8-bit floating point spec).
//
// quantize: codes = E4M3 / E5M2 of clamp(x * scale, -max, max), round to
// nearest even (the hardware conversion; the clamp makes overflow saturate,
// which the conversion alone turns into NaN), and amax = max |x| (an
// unsigned-integer max over the float bits of non-negative values: exact and
// independent of the order the workgroups finish in).
// update: the new amax enters the history (newest first, oldest dropped);
// scale = fmt_max / max(history) / 2^margin while that max is positive and
// finite, else unchanged; descale = 1 / scale.
#include "launch.h"

namespace sdpa {

__global__ void fp8_amax_clear_kernel(float* amax) {
  if (threadIdx.x == 0) amax[0] = 0.0f;
}

// Eight consecutive elements of x as float (elements at or past n read 0).
template <bool BF16_IN>
__device__ __forceinline__ void fp8_load8(const void* __restrict__ x, size_t n, size_t i0, float (&v)[8]) {
  const bool whole = i0 + 8 <= n;
  if constexpr (BF16_IN) {
    const uint16_t* xs = static_cast<const uint16_t*>(x) + i0;
    if (whole) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(xs);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[2 * e] = bf16_lo(w[e]);
        v[2 * e + 1] = bf16_hi(w[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = i0 + e < n ? __uint_as_float((uint32_t)xs[e] << 16) : 0.0f;
    }
  } else {
    const float* xs = static_cast<const float*>(x) + i0;
    if (whole) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(xs), b = *reinterpret_cast<const f32x4*>(xs + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = a[e];
        v[4 + e] = b[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = i0 + e < n ? xs[e] : 0.0f;
    }
  }
}

// Codes of eight values (saturated, round to nearest even) and their max |x|.
template <bool E5>
__device__ __forceinline__ void fp8_store8(const float (&v)[8], float sc, size_t n, size_t i0,
                                           uint8_t* __restrict__ out, float& mx) {
  constexpr float kMax = E5 ? 57344.0f : 448.0f;
  uint32_t wd[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    float y[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mx = fmaxf(mx, fabsf(v[4 * q + e]));
      y[e] = fminf(fmaxf(v[4 * q + e] * sc, -kMax), kMax);
    }
    int word;
    if constexpr (E5) {
      word = __builtin_amdgcn_cvt_pk_bf8_f32(y[0], y[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_bf8_f32(y[2], y[3], word, true);
    } else {
      word = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], word, true);
    }
    wd[q] = (uint32_t)word;
  }
  if (i0 + 8 <= n) {
    *reinterpret_cast<u32x2*>(out + i0) = u32x2{wd[0], wd[1]};
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (i0 + e < n) out[i0 + e] = (uint8_t)(wd[e >> 2] >> (8 * (e & 3)));
  }
}

// Grid-stride over groups of eight elements, four groups in flight per
// thread; one atomic max per workgroup (the grid is capped, so the atomics on
// the single amax word stay few).
template <bool E5, bool BF16_IN>
__global__ __launch_bounds__(256) void fp8_quantize_kernel(const void* __restrict__ x, size_t n,
                                                           const float* scale, uint8_t* __restrict__ out,
                                                           float* amax) {
  constexpr int U = 4;
  __shared__ float red[4];
  const float sc = scale[0];
  const size_t n_groups = (n + 7) / 8;
  const size_t stride = (size_t)gridDim.x * 256;
  float mx = 0.0f;
  for (size_t g = (size_t)blockIdx.x * 256 + threadIdx.x; g < n_groups; g += U * stride) {
    float v[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t gi = g + u * stride;
      if (gi < n_groups) fp8_load8<BF16_IN>(x, n, gi * 8, v[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t gi = g + u * stride;
      if (gi < n_groups) fp8_store8<E5>(v[u], sc, n, gi * 8, out, mx);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    atomicMax(reinterpret_cast<unsigned int*>(amax), __float_as_uint(mx));
  }
}

template __global__ void fp8_quantize_kernel<false, false>(const void*, size_t, const float*, uint8_t*, float*);
template __global__ void fp8_quantize_kernel<false, true>(const void*, size_t, const float*, uint8_t*, float*);
template __global__ void fp8_quantize_kernel<true, false>(const void*, size_t, const float*, uint8_t*, float*);
template __global__ void fp8_quantize_kernel<true, true>(const void*, size_t, const float*, uint8_t*, float*);

__global__ __launch_bounds__(256) void fp8_update_scale_kernel(float* history, int len, const float* new_amax,
                                                               float fmt_max, float margin_factor, float* scale,
                                                               float* descale) {
  __shared__ float old[kFp8MaxHistory];
  __shared__ float red[256];
  const int t = threadIdx.x;
  for (int i = t; i < len; i += 256) old[i] = history[i];
  __syncthreads();
  float mx = 0.0f;
  bool bad = false;  // a NaN or infinity in the new history
  for (int i = t; i < len; i += 256) {
    const float v = i == 0 ? new_amax[0] : old[i - 1];
    history[i] = v;
    bad |= !isfinite(v);
    mx = fmaxf(mx, v);
  }
  red[t] = bad ? __builtin_inff() : mx;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (t < w) red[t] = fmaxf(red[t], red[t + w]);
    __syncthreads();
  }
  if (t == 0) {
    const float amax = red[0];
    float s = scale[0];
    if (amax > 0.0f && isfinite(amax)) s = fmt_max / amax / margin_factor;
    scale[0] = s;
    descale[0] = 1.0f / s;
  }
}

hipError_t launch_fp8_quantize(const void* x, int bf16_in, size_t n, int e5m2, const float* scale, uint8_t* out,
                               float* amax, hipStream_t stream) {
  hipLaunchKernelGGL(fp8_amax_clear_kernel, dim3(1), dim3(64), 0, stream, amax);
  if (n == 0) return hipGetLastError();
  const size_t blocks = (n + 8 * 256 - 1) / (8 * 256);
  const dim3 grid((unsigned)(blocks < 1024 ? blocks : 1024));
  if (e5m2) {
    if (bf16_in) hipLaunchKernelGGL((fp8_quantize_kernel<true, true>), grid, dim3(256), 0, stream, x, n, scale, out, amax);
    else hipLaunchKernelGGL((fp8_quantize_kernel<true, false>), grid, dim3(256), 0, stream, x, n, scale, out, amax);
  } else {
    if (bf16_in) hipLaunchKernelGGL((fp8_quantize_kernel<false, true>), grid, dim3(256), 0, stream, x, n, scale, out, amax);
    else hipLaunchKernelGGL((fp8_quantize_kernel<false, false>), grid, dim3(256), 0, stream, x, n, scale, out, amax);
  }
  return hipGetLastError();
}

hipError_t launch_fp8_update_scale(float* history, int len, const float* amax, float fmt_max, int margin,
                                   float* scale, float* descale, hipStream_t stream) {
  hipLaunchKernelGGL(fp8_update_scale_kernel, dim3(1), dim3(256), 0, stream, history, len, amax, fmt_max,
                     ldexpf(1.0f, margin), scale, descale);
  return hipGetLastError();
}

}  // namespace sdpa
