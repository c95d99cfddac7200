// Mask-engine probes: run the kernels' own integer mask code on the device so
// tests can compare its decisions bit for bit with an independent mask; the
// same for the dropout keep decisions of the device generator.
#include "dropout.h"
#include "launch.h"

namespace sdpa {

__global__ void debug_tile_map_kernel(KArgs a, int bm, int bn, int nqt, int nkt, int8_t* out) {
  const int b = blockIdx.y, qt = blockIdx.x;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  for (int kt = threadIdx.x; kt < nkt; kt += blockDim.x)
    out[((size_t)b * nqt + qt) * nkt + kt] = (int8_t)tile_class(m, qt * bm, bm, kt * bn, bn);
}

__global__ void debug_mask_probe_kernel(KArgs a, uint8_t* out) {
  const int b = blockIdx.y, i = blockIdx.x;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  for (int j = threadIdx.x; j < a.S; j += blockDim.x)
    out[((size_t)b * a.S + i) * a.S + j] = visible(m, i, j) ? 1 : 0;
}

// out[b][h][i][j] = 1 iff pair (i, j) of batch b, query head h is kept
// (every pair, visible or not); grid (S, Hq, B).
__global__ void debug_dropout_mask_kernel(KArgs a, uint8_t* out) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const DropGen dg = drop_gen(a);
  for (int j = threadIdx.x; j < a.S; j += blockDim.x)
    out[(((size_t)b * a.Hq + h) * a.S + i) * a.S + j] = drop_keep_pair(dg, b * a.Hq + h, i, j) ? 1 : 0;
}

hipError_t launch_debug_dropout_mask(const KArgs& a, uint8_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(debug_dropout_mask_kernel, dim3(a.S, a.Hq, a.B), dim3(256), 0, stream, a, out);
  return hipGetLastError();
}

hipError_t launch_debug_tile_map(const KArgs& a, int bm, int bn, int8_t* out, hipStream_t stream) {
  const int nqt = (a.S + bm - 1) / bm, nkt = (a.S + bn - 1) / bn;
  hipLaunchKernelGGL(debug_tile_map_kernel, dim3(nqt, a.B), dim3(256), 0, stream, a, bm, bn, nqt, nkt, out);
  return hipGetLastError();
}

hipError_t launch_debug_mask_probe(const KArgs& a, uint8_t* out, hipStream_t stream) {
  hipLaunchKernelGGL(debug_mask_probe_kernel, dim3(a.S, a.B), dim3(256), 0, stream, a, out);
  return hipGetLastError();
}

}  // namespace sdpa
