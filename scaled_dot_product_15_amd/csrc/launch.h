// Internal launcher declarations (host side of the kernels).
#pragma once

#include <hip/hip_runtime.h>

#include "attn_common.h"
#include "sdpa_attn.h"

namespace sdpa {

// Rows per block of the backward pre-pass; also the chunk of the d(sink)
// partial sums.
constexpr int kPreRows = 64;      // rows per block of the fp32 pre-pass
constexpr int kDqChunkRows = 32;  // rows per sink-gradient partial of the bf16 dQ kernel

bool fwd_bf16_tiles(int dqk, int dv, int* bm, int* bn);
hipError_t launch_fwd_bf16(const KArgs& a, int dqk, int dv, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16(const KArgs& a, int dqk, int dv, hipStream_t stream);
// Query-head splits of a GQA group in the bf16 dK/dV kernel: the smallest
// divisor d of G for which the grid of key tiles x batches x kv heads x d
// holds at least kDkdvMinGrid workgroups and one workgroup walks at most
// kDkdvMaxBlocks 32-row blocks (long workgroups leave a tail of idle CUs);
// G if none does; then lowered to the largest divisor whose fp32 partials
// fit in kDkdvMaxPartialBytes (1 if none).  wl, wr: windows normalised to
// -1 or < S.
constexpr int kDkdvKeyTile = 128;
#ifndef SDPA_DKDV_MIN_GRID
#define SDPA_DKDV_MIN_GRID 1024
#endif
#ifndef SDPA_DKDV_MAX_BLOCKS
#define SDPA_DKDV_MAX_BLOCKS 512
#endif
constexpr int kDkdvMinGrid = SDPA_DKDV_MIN_GRID;
constexpr long long kDkdvMaxBlocks = SDPA_DKDV_MAX_BLOCKS;
constexpr long long kDkdvMaxPartialBytes = 1ll << 30;
int dkdv_head_splits(int B, int S, int Hkv, int G, bool causal, int wl, int wr, int dqk, int dv);
// dK / dV = sum over the splits of the partials, in split order (bf16 out).
hipError_t launch_dkdv_split_reduce(const KArgs& a, int dqk, int dv, hipStream_t stream);
hipError_t launch_bwd_dq_bf16(const KArgs& a, int dqk, int dv, hipStream_t stream);
// dQ from the dS blocks the dK/dV kernel stored in a.ds (a.ds_nkt, a.ds_nqb
// set; head dims 64/64 or 128/128).
hipError_t launch_bwd_dq_ds_bf16(const KArgs& a, int dqk, int dv, hipStream_t stream);
// Gradient of the attention bias (needs the pre-pass's delta and LSE * log2 e).
int dbias_key_chunks(int n_mats, int n_qt, int n_kt);
hipError_t launch_bwd_dbias_bf16(const KArgs& a, int dqk, int dv, hipStream_t stream);
// dBias from the stored dS blocks (the stored-dS backward: a.ds set, after the
// dK/dV kernel).
hipError_t launch_dbias_from_ds(const KArgs& a, hipStream_t stream);

// FP8 forward (E4M3 Q, K, V): V^T pre-pass into a.vt, then the two-pass kernel.
size_t fp8_vt_bytes(int B, int S, int Hkv, int dv);
hipError_t launch_fwd_fp8(const KArgs& a, int dqk, int dv, hipStream_t stream);
// FP8 codes [rows, heads, d] per batch -> [B, heads, d, a.s_pad] (positions of
// each 64-group in fp8_key_slot order, zero past the valid length).
hipError_t launch_fp8_transpose(const KArgs& a, const void* src, int heads, uint8_t* dst, int d, hipStream_t stream);
// FP8 backward (E4M3 Q, K, V, E5M2 dO): pre-pass, transposes of K, Q, dO into
// a.kt_t / a.qt_t / a.dot_t, dQ and dK/dV kernels, sink-gradient reduce.
size_t fp8_bwd_transposed_bytes(int B, int S, int Hq, int Hkv, int d);
hipError_t launch_bwd_fp8(const KArgs& a, int dqk, int dv, hipStream_t stream);
// FP8 per-tensor scaling.
hipError_t launch_fp8_quantize(const void* x, int bf16_in, size_t n, int e5m2, const float* scale, uint8_t* out,
                               float* amax, hipStream_t stream);
constexpr int kFp8MaxHistory = 4096;
hipError_t launch_fp8_update_scale(float* history, int len, const float* amax, float fmt_max, int margin,
                                   float* scale, float* descale, hipStream_t stream);

bool fwd_f32_tiles(int dqk, int dv, int* bm, int* bn);
hipError_t launch_fwd_f32(const KArgs& a, int dqk, int dv, hipStream_t stream);
hipError_t launch_bwd_dkdv_f32(const KArgs& a, int dqk, int dv, hipStream_t stream);
hipError_t launch_bwd_dq_f32(const KArgs& a, int dqk, int dv, hipStream_t stream);

// delta = rowsum(dO * O) and d(sink) partials; dtype 0 = f32, 1 = bf16.
hipError_t launch_bwd_pre(const KArgs& a, int dtype, int dv, hipStream_t stream);
// d_softmax_offset[h] = sum over batches and chunks, fixed order.
hipError_t launch_dz_reduce(const KArgs& a, hipStream_t stream);

// Attention bias of attn_bwd_bias: [batch, heads, S, S] and its gradient
// (d_bias may be NULL).
struct BiasArgs {
  const void* bias;
  void* d_bias;
  int32_t batch, heads;
};
// The backward of attn_bwd / attn_bwd_stage / attn_bwd_bias (stage 0 = all
// stages; bias only with stage 0, else NULL) with the workspace at
// `workspace`: host checks, then launches on `stream`.
int bwd_run(int stage, const attn_params* p, const void* q, const void* k, const void* v, const void* o,
            const void* d_o, const float* lse, const float* softmax_offset, const int32_t* seqlens,
            const int32_t* seq_offsets, void* dq, void* dk, void* dv, float* d_softmax_offset, void* workspace,
            size_t workspace_bytes, void* stream, const BiasArgs* bias);

hipError_t launch_debug_tile_map(const KArgs& a, int bm, int bn, int8_t* out, hipStream_t stream);
hipError_t launch_debug_mask_probe(const KArgs& a, uint8_t* out, hipStream_t stream);
hipError_t launch_debug_dropout_mask(const KArgs& a, uint8_t* out, hipStream_t stream);

}  // namespace sdpa
