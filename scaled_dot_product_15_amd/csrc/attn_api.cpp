// Host side of the C ABI declared in include/sdpa_attn.h: argument checks,
// workspace layout, kernel choice and launches on the caller's stream.
// Nothing here allocates device memory or synchronises.
#include <math.h>
#include <stdint.h>

#include "launch.h"
#include "sdpa_attn.h"

using namespace sdpa;

namespace {

bool supported(const attn_params* p) {
  // A negative scale is a valid problem; the kernels take each row's running
  // max on unscaled scores and multiply it by the scale, which needs scale >= 0.
  if (p->scale_factor < 0.0f) return false;
  if (p->dtype == ATTN_FP8) {
    // E4M3 forward: head dims 64 or 128, no dropout.
    return p->head_dim_qk == p->head_dim_v && (p->head_dim_qk == 64 || p->head_dim_qk == 128) &&
           p->dropout_p == 0.0f;
  }
  int bm, bn;
  if (p->dtype == ATTN_BF16) return fwd_bf16_tiles(p->head_dim_qk, p->head_dim_v, &bm, &bn);
  return fwd_f32_tiles(p->head_dim_qk, p->head_dim_v, &bm, &bn);
}

int check_fields(const attn_params* p) {
  if (!p) return ATTN_ERR_INVALID_ARG;
  if (p->batch < 1 || p->seqlen < 1 || p->num_heads < 1 || p->num_gqa_groups < 1) return ATTN_ERR_INVALID_ARG;
  if (p->num_heads % p->num_gqa_groups != 0) return ATTN_ERR_INVALID_ARG;
  if (p->head_dim_qk < 1 || p->head_dim_v < 1) return ATTN_ERR_INVALID_ARG;
  if (p->dtype != ATTN_F32 && p->dtype != ATTN_BF16 && p->dtype != ATTN_FP8) return ATTN_ERR_INVALID_ARG;
  if (p->mask_type != ATTN_MASK_NONE && p->mask_type != ATTN_MASK_CAUSAL) return ATTN_ERR_INVALID_ARG;
  if (p->window_left < -1 || p->window_right < -1) return ATTN_ERR_INVALID_ARG;
  if (!isfinite(p->scale_factor)) return ATTN_ERR_INVALID_ARG;
  if (p->softmax_type < ATTN_SOFTMAX_VANILLA || p->softmax_type > ATTN_SOFTMAX_LEARNABLE) return ATTN_ERR_INVALID_ARG;
  if (!(p->dropout_p >= 0.0f && p->dropout_p < 1.0f)) return ATTN_ERR_INVALID_ARG;  // also rejects NaN
  // Kernels index rows with 32-bit (batch * S + i) and launch one-dimensional
  // grids of B * heads * tiles workgroups.
  const long long rows = (long long)p->batch * p->seqlen;
  const long long grid = (long long)p->batch * p->num_heads * ((p->seqlen + 63) / 64);
  if (rows > 0x7fffffffLL || grid > 0x7fffffffLL) return ATTN_ERR_INVALID_ARG;
  // Kernels address one batch of one tensor with 32-bit byte offsets.
  const long long dmax = p->head_dim_qk > p->head_dim_v ? p->head_dim_qk : p->head_dim_v;
  if ((long long)p->seqlen * p->num_heads * dmax * 4 > 0xffffffffLL) return ATTN_ERR_INVALID_ARG;
  return ATTN_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// Rows per sink-gradient partial: the bf16 dQ kernel writes one per wave
// (32 rows), the fp32 pre-pass one per 64-row block; the workspace holds the
// larger count.
int chunk_rows(const attn_params* p) { return p->dtype == ATTN_F32 ? kPreRows : kDqChunkRows; }
int n_chunks(const attn_params* p) { return (p->seqlen + chunk_rows(p) - 1) / chunk_rows(p); }
int max_chunks(const attn_params* p) { return (p->seqlen + kDqChunkRows - 1) / kDqChunkRows; }
size_t delta_bytes(const attn_params* p) { return align256((size_t)p->batch * p->num_heads * p->seqlen * sizeof(float)); }
size_t dz_bytes(const attn_params* p) { return align256((size_t)p->batch * p->num_heads * max_chunks(p) * sizeof(float)); }
// bf16 dK/dV: query-head splits of a GQA group (fp32 partials in the workspace when > 1).
int kv_splits(const attn_params* p) {
  if (p->dtype == ATTN_F32) return 1;  // bf16 and FP8 dK/dV kernels split a GQA group's heads
  return dkdv_head_splits(p->batch, p->seqlen, p->num_gqa_groups, p->num_heads / p->num_gqa_groups,
                          p->mask_type == ATTN_MASK_CAUSAL, normalise_window(p->window_left, p->seqlen),
                          normalise_window(p->window_right, p->seqlen), p->head_dim_qk, p->head_dim_v);
}
size_t kv_part_bytes(const attn_params* p) {
  const int ns = kv_splits(p);
  if (ns == 1) return 0;
  return align256((size_t)ns * p->batch * p->seqlen * p->num_gqa_groups * (p->head_dim_qk + p->head_dim_v) *
                  sizeof(float));
}

// bf16 backward with stored dS: every bf16 head dim pair, with or without
// dropout (the stored dS has the dropout applied, so dQ = scale dS K needs no
// random bytes).  Per (batch, head) the slabs of the 128-key tiles, back to
// back, each ds_tile_blocks blocks of 8 KiB (mask at the full length).
bool ds_eligible(const attn_params* p) { return p->dtype == ATTN_BF16; }
long long ds_head_blocks(const attn_params* p) {
  const MaskSpec m = make_mask(p->seqlen, p->seqlen, p->mask_type == ATTN_MASK_CAUSAL, p->window_left, p->window_right);
  long long n = 0;
  for (int kt = 0; kt < (p->seqlen + kDkdvKeyTile - 1) / kDkdvKeyTile; ++kt) n += ds_tile_blocks(m, kt);
  return n;
}
constexpr size_t kDsBlockBytes = 8192;  // 32 rows x 128 keys, bf16
size_t ds_bytes(const attn_params* p) {
  return align256((size_t)p->batch * p->num_heads * (size_t)ds_head_blocks(p) * kDsBlockBytes);
}

KArgs make_args(const attn_params* p) {
  KArgs a = {};
  a.B = p->batch;
  a.S = p->seqlen;
  a.Hq = p->num_heads;
  a.Hkv = p->num_gqa_groups;
  a.G = p->num_heads / p->num_gqa_groups;
  a.causal = p->mask_type == ATTN_MASK_CAUSAL;
  a.wl = normalise_window(p->window_left, p->seqlen);
  a.wr = normalise_window(p->window_right, p->seqlen);
  a.softmax_type = p->softmax_type;
  a.scale = p->scale_factor != 0.0f ? p->scale_factor : (float)(1.0 / sqrt((double)p->head_dim_qk));
  a.scale_log2 = a.scale * kLog2e;
  a.inv_scale = 1.0f / a.scale;
  a.n_chunks = n_chunks(p);
  a.n_splits = kv_splits(p);
  // Dropout: byte threshold round(256 p), kept probabilities scaled by
  // 1 / (1 - t / 256); t = 0 (p < 1/512) means no dropout.
  const double t = floor(256.0 * (double)p->dropout_p + 0.5);
  a.drop_t = t > 255.0 ? 255 : (int)t;
  a.drop_scale = (float)(1.0 / (1.0 - a.drop_t / 256.0));
  a.drop_seed_lo = p->dropout_seed_lo;
  a.drop_seed_hi = p->dropout_seed_hi;
  a.drop_offset = p->dropout_offset;
  return a;
}

// Bias arguments (attn_fwd_bias / attn_bwd_bias): an additive post-scale bias
// of shape [bias_batch, bias_heads, S, S] in the input dtype.
int check_bias(const attn_params* p, const void* bias, int32_t bias_batch, int32_t bias_heads) {
  if (!bias) return ATTN_ERR_INVALID_ARG;
  if (bias_batch != 1 && bias_batch != p->batch) return ATTN_ERR_INVALID_ARG;
  if (bias_heads != 1 && bias_heads != p->num_heads) return ATTN_ERR_INVALID_ARG;
  if (p->dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  const bool dims = (p->head_dim_qk == 64 && p->head_dim_v == 64) || (p->head_dim_qk == 128 && p->head_dim_v == 128);
  if (!dims) return ATTN_ERR_UNSUPPORTED;
  // Kernels address one [S, S] bias matrix with 32-bit byte offsets, copy
  // 16-byte pieces of its rows (rows of S * 2 bytes, S a multiple of 8, on a
  // 16-byte aligned base) and add bias / scale to the unscaled scores.
  if ((long long)p->seqlen * p->seqlen * 2 > 0xffffffffLL) return ATTN_ERR_UNSUPPORTED;
  if (p->seqlen % 8 != 0) return ATTN_ERR_UNSUPPORTED;
  if ((reinterpret_cast<uintptr_t>(bias) & 15) != 0) return ATTN_ERR_INVALID_ARG;
  const KArgs a = make_args(p);
  if (!isfinite(a.inv_scale)) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

void set_bias(KArgs& a, const void* bias, void* d_bias, int32_t bias_batch, int32_t bias_heads) {
  a.bias = bias;
  a.d_bias = d_bias;
  a.bias_b = bias_batch;
  a.bias_h = bias_heads;
}

MaskSpec host_mask(const attn_params* p, int L) {
  return make_mask(L, p->seqlen, p->mask_type == ATTN_MASK_CAUSAL, p->window_left, p->window_right);
}

int hip_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

}  // namespace

extern "C" {

int attn_validate(const attn_params* p) {
  const int rc = check_fields(p);
  if (rc != ATTN_OK) return rc;
  return supported(p) ? ATTN_OK : ATTN_ERR_UNSUPPORTED;
}

size_t attn_fwd_workspace_size(const attn_params* p) {
  if (attn_validate(p) != ATTN_OK) return 0;
  if (p->dtype != ATTN_FP8) return 0;
  return align256(fp8_vt_bytes(p->batch, p->seqlen, p->num_gqa_groups, p->head_dim_v));
}

size_t attn_bwd_ds_workspace_size(const attn_params* p) {
  if (attn_validate(p) != ATTN_OK || !ds_eligible(p)) return 0;
  // The kernels index a head's blocks with 32-bit integers.
  if (ds_head_blocks(p) > 0x7fffffffLL) return 0;
  return attn_bwd_workspace_size(p) + ds_bytes(p);
}

size_t attn_bwd_workspace_size(const attn_params* p) {
  if (attn_validate(p) != ATTN_OK) return 0;
  if (p->dtype == ATTN_FP8)
    return 2 * delta_bytes(p) + dz_bytes(p) +
           align256(fp8_bwd_transposed_bytes(p->batch, p->seqlen, p->num_heads, p->num_gqa_groups, p->head_dim_qk)) +
           kv_part_bytes(p);
  return 2 * delta_bytes(p) + dz_bytes(p) + kv_part_bytes(p);
}

}  // extern "C"

namespace {

int fwd_run(const attn_params* p, const void* q, const void* k, const void* v, const void* bias, int32_t bias_batch,
            int32_t bias_heads, const float* softmax_offset, const int32_t* seqlens, const int32_t* seq_offsets,
            void* o, float* lse, void* stream) {
  const int rc = attn_validate(p);
  if (rc != ATTN_OK) return rc;
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_INVALID_ARG;
  if (p->softmax_type == ATTN_SOFTMAX_LEARNABLE && !softmax_offset) return ATTN_ERR_INVALID_ARG;
  if (bias) {
    const int rb = check_bias(p, bias, bias_batch, bias_heads);
    if (rb != ATTN_OK) return rb;
  }
  KArgs a = make_args(p);
  if (bias) set_bias(a, bias, nullptr, bias_batch, bias_heads);
  if (p->dtype == ATTN_FP8) return ATTN_ERR_UNSUPPORTED;  // through attn_fwd_fp8 only
  a.q = q;
  a.k = k;
  a.v = v;
  a.softmax_offset = softmax_offset;
  a.seqlens = seqlens;
  a.seq_offsets = seq_offsets;
  a.out_o = o;
  a.out_lse = lse;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (p->dtype == ATTN_BF16) return hip_status(launch_fwd_bf16(a, p->head_dim_qk, p->head_dim_v, s));
  return hip_status(launch_fwd_f32(a, p->head_dim_qk, p->head_dim_v, s));
}

}  // namespace

extern "C" {

int attn_fwd(const attn_params* p, const void* q, const void* k, const void* v, const float* softmax_offset,
             const int32_t* seqlens, const int32_t* seq_offsets, void* o, float* lse, void* workspace,
             size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (p && p->dtype == ATTN_FP8) return check_fields(p) == ATTN_OK ? ATTN_ERR_UNSUPPORTED : ATTN_ERR_INVALID_ARG;
  return fwd_run(p, q, k, v, nullptr, 0, 0, softmax_offset, seqlens, seq_offsets, o, lse, stream);
}

int attn_fwd_bias(const attn_params* p, const void* q, const void* k, const void* v, const void* bias,
                  int32_t bias_batch, int32_t bias_heads, const float* softmax_offset, const int32_t* seqlens,
                  const int32_t* seq_offsets, void* o, float* lse, void* workspace, size_t workspace_bytes,
                  void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!bias) return ATTN_ERR_INVALID_ARG;
  return fwd_run(p, q, k, v, bias, bias_batch, bias_heads, softmax_offset, seqlens, seq_offsets, o, lse, stream);
}

}  // extern "C"

namespace sdpa {

int bwd_run(int stage, const attn_params* p, const void* q, const void* k, const void* v, const void* o,
               const void* d_o, const float* lse, const float* softmax_offset, const int32_t* seqlens,
               const int32_t* seq_offsets, void* dq, void* dk, void* dv, float* d_softmax_offset, void* workspace,
               size_t workspace_bytes, void* stream, const BiasArgs* bias) {
  if (stage < 0 || stage > ATTN_BWD_STAGE_OFFSET_GRAD) return ATTN_ERR_INVALID_ARG;
  const int rc = attn_validate(p);
  if (rc != ATTN_OK) return rc;
  if (p->dtype == ATTN_FP8) return ATTN_ERR_UNSUPPORTED;  // FP8: through attn_bwd_fp8 only
  if (!q || !k || !v || !o || !d_o || !lse || !dq || !dk || !dv) return ATTN_ERR_INVALID_ARG;
  if (p->softmax_type == ATTN_SOFTMAX_LEARNABLE && (!softmax_offset || !d_softmax_offset)) return ATTN_ERR_INVALID_ARG;
  if (p->softmax_type == ATTN_SOFTMAX_VANILLA && d_softmax_offset) return ATTN_ERR_INVALID_ARG;
  if (!workspace) return ATTN_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return ATTN_ERR_INVALID_ARG;
  if (workspace_bytes < attn_bwd_workspace_size(p)) return ATTN_ERR_WORKSPACE;
  if (bias) {
    if (stage != 0) return ATTN_ERR_INVALID_ARG;
    const int rb = check_bias(p, bias->bias, bias->batch, bias->heads);
    if (rb != ATTN_OK) return rb;
    if ((reinterpret_cast<uintptr_t>(bias->d_bias) & 15) != 0) return ATTN_ERR_INVALID_ARG;
  }
  KArgs a = make_args(p);
  if (bias) set_bias(a, bias->bias, bias->d_bias, bias->batch, bias->heads);
  // With room for the dS blocks: pre-pass, dK/dV storing dS, dQ from the
  // stored dS (and dBias summed from it) -- stages 1, 3, 2, 4.  Otherwise
  // 1, 2, 3, 4, the bf16 dQ kernel running the pre-pass itself.
  const size_t ds_ws = attn_bwd_ds_workspace_size(p);
  const bool use_ds = ds_ws > 0 && workspace_bytes >= ds_ws;
  // A bias with one matrix per (batch, head) has dBias = dS: on the
  // recomputing path the dQ kernel writes it (its dS values, zeros
  // elsewhere) and no separate pass runs.
  a.dbias_direct = !use_ds && bias && bias->d_bias && bias->batch == p->batch && bias->heads == p->num_heads;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.d_o = d_o;
  a.lse = lse;
  a.softmax_offset = softmax_offset;
  a.seqlens = seqlens;
  a.seq_offsets = seq_offsets;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.d_offset = d_softmax_offset;
  a.delta = static_cast<float*>(workspace);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(workspace) + delta_bytes(p));
  a.dz_partial = reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * delta_bytes(p));
  a.kv_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + 2 * delta_bytes(p) + dz_bytes(p));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf16 = p->dtype == ATTN_BF16;
  const int dqk = p->head_dim_qk, dvd = p->head_dim_v;
  if (use_ds) {
    a.ds = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + attn_bwd_workspace_size(p));
    a.ds_head_blocks = (int)ds_head_blocks(p);
    a.n_chunks = (p->seqlen + kPreRows - 1) / kPreRows;  // sink-gradient partials of the pre-pass
  }
  if ((stage == 0 || stage == ATTN_BWD_STAGE_PREPROCESS) && (!bf16 || use_ds)) {
    if (launch_bwd_pre(a, bf16 ? 1 : 0, dvd, s) != hipSuccess) return ATTN_ERR_HIP;
  }
  auto run_dq = [&]() {
    if (use_ds) return launch_bwd_dq_ds_bf16(a, dqk, dvd, s);
    return bf16 ? launch_bwd_dq_bf16(a, dqk, dvd, s) : launch_bwd_dq_f32(a, dqk, dvd, s);
  };
  auto run_dkdv = [&]() {
    hipError_t e = bf16 ? launch_bwd_dkdv_bf16(a, dqk, dvd, s) : launch_bwd_dkdv_f32(a, dqk, dvd, s);
    if (e == hipSuccess && a.n_splits > 1) e = launch_dkdv_split_reduce(a, dqk, dvd, s);
    return e;
  };
  if (stage == 0 && use_ds) {
    if (run_dkdv() != hipSuccess || run_dq() != hipSuccess) return ATTN_ERR_HIP;
  } else {
    if ((stage == 0 || stage == ATTN_BWD_STAGE_DQ) && run_dq() != hipSuccess) return ATTN_ERR_HIP;
    if ((stage == 0 || stage == ATTN_BWD_STAGE_DKDV) && run_dkdv() != hipSuccess) return ATTN_ERR_HIP;
  }
  if (stage == 0 && a.bias && a.d_bias && !a.dbias_direct) {
    if ((use_ds ? launch_dbias_from_ds(a, s) : launch_bwd_dbias_bf16(a, dqk, dvd, s)) != hipSuccess)
      return ATTN_ERR_HIP;
  }
  if ((stage == 0 || stage == ATTN_BWD_STAGE_OFFSET_GRAD) && d_softmax_offset &&
      p->softmax_type != ATTN_SOFTMAX_VANILLA) {
    if (launch_dz_reduce(a, s) != hipSuccess) return ATTN_ERR_HIP;
  }
  return ATTN_OK;
}

}  // namespace sdpa

extern "C" {

int attn_bwd(const attn_params* p, const void* q, const void* k, const void* v, const void* o, const void* d_o,
             const float* lse, const float* softmax_offset, const int32_t* seqlens, const int32_t* seq_offsets,
             void* dq, void* dk, void* dv, float* d_softmax_offset, void* workspace, size_t workspace_bytes,
             void* stream) {
  return bwd_run(0, p, q, k, v, o, d_o, lse, softmax_offset, seqlens, seq_offsets, dq, dk, dv, d_softmax_offset,
                    workspace, workspace_bytes, stream, nullptr);
}

int attn_bwd_bias(const attn_params* p, const void* q, const void* k, const void* v, const void* o, const void* d_o,
                  const float* lse, const void* bias, int32_t bias_batch, int32_t bias_heads, void* d_bias,
                  const float* softmax_offset, const int32_t* seqlens, const int32_t* seq_offsets, void* dq, void* dk,
                  void* dv, float* d_softmax_offset, void* workspace, size_t workspace_bytes, void* stream) {
  if (!bias) return ATTN_ERR_INVALID_ARG;
  const BiasArgs ba = {bias, d_bias, bias_batch, bias_heads};
  return bwd_run(0, p, q, k, v, o, d_o, lse, softmax_offset, seqlens, seq_offsets, dq, dk, dv, d_softmax_offset,
                 workspace, workspace_bytes, stream, &ba);
}

int attn_bwd_stage(int stage, const attn_params* p, const void* q, const void* k, const void* v, const void* o,
                   const void* d_o, const float* lse, const float* softmax_offset, const int32_t* seqlens,
                   const int32_t* seq_offsets, void* dq, void* dk, void* dv, float* d_softmax_offset,
                   void* workspace, size_t workspace_bytes, void* stream) {
  if (stage < ATTN_BWD_STAGE_PREPROCESS) return ATTN_ERR_INVALID_ARG;
  return bwd_run(stage, p, q, k, v, o, d_o, lse, softmax_offset, seqlens, seq_offsets, dq, dk, dv,
                    d_softmax_offset, workspace, workspace_bytes, stream, nullptr);
}

int attn_fwd_fp8(const attn_params* p, const void* q, const void* k, const void* v, const float* descale_qkv,
                 const float* softmax_offset, const int32_t* seqlens, const int32_t* seq_offsets, void* o, float* lse,
                 void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = attn_validate(p);
  if (rc != ATTN_OK) return rc;
  if (p->dtype != ATTN_FP8) return ATTN_ERR_INVALID_ARG;
  if (!q || !k || !v || !descale_qkv || !o || !lse) return ATTN_ERR_INVALID_ARG;
  if (p->softmax_type == ATTN_SOFTMAX_LEARNABLE && !softmax_offset) return ATTN_ERR_INVALID_ARG;
  // 16-byte row pieces of Q, K, V are read directly.
  if (((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) | reinterpret_cast<uintptr_t>(v)) & 15) != 0)
    return ATTN_ERR_INVALID_ARG;
  if (!workspace) return ATTN_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return ATTN_ERR_INVALID_ARG;
  if (workspace_bytes < attn_fwd_workspace_size(p)) return ATTN_ERR_WORKSPACE;
  KArgs a = make_args(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.fp8_descale = descale_qkv;
  a.softmax_offset = softmax_offset;
  a.seqlens = seqlens;
  a.seq_offsets = seq_offsets;
  a.out_o = o;
  a.out_lse = lse;
  a.vt = static_cast<uint8_t*>(workspace);
  return hip_status(launch_fwd_fp8(a, p->head_dim_qk, p->head_dim_v, static_cast<hipStream_t>(stream)));
}

int attn_bwd_fp8(const attn_params* p, const void* q, const void* k, const void* v, const void* o, const void* d_o,
                 const float* lse, const float* descale_qkvdo, const float* ds_scale, float* amax_ds,
                 const float* softmax_offset, const int32_t* seqlens, const int32_t* seq_offsets, void* dq, void* dk,
                 void* dv, float* d_softmax_offset, void* workspace, size_t workspace_bytes, void* stream) {
  const int rc = attn_validate(p);
  if (rc != ATTN_OK) return rc;
  if (p->dtype != ATTN_FP8) return ATTN_ERR_INVALID_ARG;
  if (!q || !k || !v || !o || !d_o || !lse || !descale_qkvdo || !ds_scale || !amax_ds || !dq || !dk || !dv)
    return ATTN_ERR_INVALID_ARG;
  if (p->softmax_type == ATTN_SOFTMAX_LEARNABLE && (!softmax_offset || !d_softmax_offset)) return ATTN_ERR_INVALID_ARG;
  if (p->softmax_type == ATTN_SOFTMAX_VANILLA && d_softmax_offset) return ATTN_ERR_INVALID_ARG;
  // 16-byte row pieces of Q, K, V, dO are read directly; O rows in 8- or 16-byte pieces.
  const uintptr_t in = reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(k) |
                       reinterpret_cast<uintptr_t>(v) | reinterpret_cast<uintptr_t>(d_o) |
                       reinterpret_cast<uintptr_t>(o);
  if ((in & 15) != 0) return ATTN_ERR_INVALID_ARG;
  if (!workspace) return ATTN_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return ATTN_ERR_INVALID_ARG;
  if (workspace_bytes < attn_bwd_workspace_size(p)) return ATTN_ERR_WORKSPACE;
  KArgs a = make_args(p);
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.d_o = d_o;
  a.lse = lse;
  a.fp8_descale = descale_qkvdo;
  a.ds_scale = ds_scale;
  a.amax_out = amax_ds;
  a.softmax_offset = softmax_offset;
  a.seqlens = seqlens;
  a.seq_offsets = seq_offsets;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.d_offset = d_softmax_offset;
  char* ws = static_cast<char*>(workspace);
  a.delta = reinterpret_cast<float*>(ws);
  a.lse2 = reinterpret_cast<float*>(ws + delta_bytes(p));
  a.dz_partial = reinterpret_cast<float*>(ws + 2 * delta_bytes(p));
  // K^T, Q^T, dO^T: [B, heads, D, S_pad] codes each
  const size_t s_pad = (size_t)((p->seqlen + 63) / 64) * 64, d = (size_t)p->head_dim_qk;
  a.kt_t = reinterpret_cast<uint8_t*>(ws + 2 * delta_bytes(p) + dz_bytes(p));
  a.qt_t = a.kt_t + (size_t)p->batch * p->num_gqa_groups * d * s_pad;
  a.dot_t = a.qt_t + (size_t)p->batch * p->num_heads * d * s_pad;
  // fp32 partial dK, dV of the query-head splits (when the split rule asks for them)
  a.kv_part = reinterpret_cast<float*>(ws + 2 * delta_bytes(p) + dz_bytes(p) +
                                       align256(fp8_bwd_transposed_bytes(p->batch, p->seqlen, p->num_heads,
                                                                         p->num_gqa_groups, p->head_dim_qk)));
  return hip_status(launch_bwd_fp8(a, p->head_dim_qk, p->head_dim_v, static_cast<hipStream_t>(stream)));
}

int attn_fp8_quantize(const void* x, int32_t x_dtype, size_t n, int32_t fmt, const float* scale, uint8_t* out,
                      float* amax, void* stream) {
  if (x_dtype != ATTN_F32 && x_dtype != ATTN_BF16) return ATTN_ERR_INVALID_ARG;
  if (fmt != ATTN_FP8_E4M3 && fmt != ATTN_FP8_E5M2) return ATTN_ERR_INVALID_ARG;
  if ((n > 0 && (!x || !out)) || !scale || !amax) return ATTN_ERR_INVALID_ARG;
  // whole 8-element groups are read and written as vectors
  const uintptr_t align = x_dtype == ATTN_BF16 ? 15 : 31;
  if ((reinterpret_cast<uintptr_t>(x) & align) != 0 || (reinterpret_cast<uintptr_t>(out) & 7) != 0)
    return ATTN_ERR_INVALID_ARG;
  return hip_status(launch_fp8_quantize(x, x_dtype == ATTN_BF16, n, fmt == ATTN_FP8_E5M2, scale, out, amax,
                                        static_cast<hipStream_t>(stream)));
}

int attn_fp8_update_scale(float* amax_history, int32_t history_len, const float* amax, int32_t fmt, int32_t margin,
                          float* scale, float* descale, void* stream) {
  if (!amax_history || !amax || !scale || !descale) return ATTN_ERR_INVALID_ARG;
  if (history_len < 1 || history_len > kFp8MaxHistory) return ATTN_ERR_INVALID_ARG;
  if (fmt != ATTN_FP8_E4M3 && fmt != ATTN_FP8_E5M2) return ATTN_ERR_INVALID_ARG;
  if (margin < 0 || margin > 64) return ATTN_ERR_INVALID_ARG;
  const float fmt_max = fmt == ATTN_FP8_E4M3 ? 448.0f : 57344.0f;
  return hip_status(launch_fp8_update_scale(amax_history, history_len, amax, fmt_max, margin, scale, descale,
                                            static_cast<hipStream_t>(stream)));
}

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID_ARG: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported: no kernel for this (dtype, head_dim_qk, head_dim_v) or a negative scale";
    case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case ATTN_ERR_HIP: return "HIP launch failed";
    case ATTN_ERR_TOO_LARGE: return "backward workspace exceeds the allocation-free scratch (64 MiB)";
    default: return "unknown status";
  }
}

int attn_fwd_tile_shape(const attn_params* p, int32_t* block_m, int32_t* block_n) {
  const int rc = attn_validate(p);
  if (rc != ATTN_OK) return rc;
  if (!block_m || !block_n) return ATTN_ERR_INVALID_ARG;
  int bm = 0, bn = 0;
  if (p->dtype == ATTN_BF16) fwd_bf16_tiles(p->head_dim_qk, p->head_dim_v, &bm, &bn);
  else if (p->dtype == ATTN_FP8) bm = 128, bn = 64;
  else fwd_f32_tiles(p->head_dim_qk, p->head_dim_v, &bm, &bn);
  *block_m = bm;
  *block_n = bn;
  return ATTN_OK;
}

int attn_debug_tile_map(const attn_params* p, const int32_t* seqlens, int32_t block_m, int32_t block_n,
                        int8_t* out, void* stream) {
  const int rc = check_fields(p);
  if (rc != ATTN_OK) return rc;
  if (!out || block_m < 1 || block_n < 1) return ATTN_ERR_INVALID_ARG;
  KArgs a = make_args(p);
  a.seqlens = seqlens;
  return hip_status(launch_debug_tile_map(a, block_m, block_n, out, static_cast<hipStream_t>(stream)));
}

int attn_debug_dropout_mask(const attn_params* p, uint8_t* out, void* stream) {
  const int rc = check_fields(p);
  if (rc != ATTN_OK) return rc;
  if (!out) return ATTN_ERR_INVALID_ARG;
  return hip_status(launch_debug_dropout_mask(make_args(p), out, static_cast<hipStream_t>(stream)));
}

int attn_debug_mask_probe(const attn_params* p, const int32_t* seqlens, uint8_t* out, void* stream) {
  const int rc = check_fields(p);
  if (rc != ATTN_OK) return rc;
  if (!out) return ATTN_ERR_INVALID_ARG;
  KArgs a = make_args(p);
  a.seqlens = seqlens;
  return hip_status(launch_debug_mask_probe(a, out, static_cast<hipStream_t>(stream)));
}

int attn_host_tile_map(const attn_params* p, const int32_t* seqlens, int32_t block_m, int32_t block_n,
                       int8_t* out) {
  const int rc = check_fields(p);
  if (rc != ATTN_OK) return rc;
  if (!out || block_m < 1 || block_n < 1) return ATTN_ERR_INVALID_ARG;
  const int S = p->seqlen, nqt = (S + block_m - 1) / block_m, nkt = (S + block_n - 1) / block_n;
  for (int b = 0; b < p->batch; ++b) {
    const MaskSpec m = host_mask(p, seqlens ? seqlens[b] : S);
    for (int qt = 0; qt < nqt; ++qt)
      for (int kt = 0; kt < nkt; ++kt)
        out[((size_t)b * nqt + qt) * nkt + kt] = (int8_t)tile_class(m, qt * block_m, block_m, kt * block_n, block_n);
  }
  return ATTN_OK;
}

int attn_host_key_range(const attn_params* p, int32_t L, int32_t i0, int32_t i1, int32_t* lo, int32_t* hi) {
  if (check_fields(p) != ATTN_OK || !lo || !hi) return 0;
  int a = 0, b = -1;
  const bool ok = key_range(host_mask(p, L), i0, i1, a, b);
  *lo = a;
  *hi = b;
  return ok ? 1 : 0;
}

int attn_host_query_range(const attn_params* p, int32_t L, int32_t j0, int32_t j1, int32_t* lo, int32_t* hi) {
  if (check_fields(p) != ATTN_OK || !lo || !hi) return 0;
  int a = 0, b = -1;
  const bool ok = query_range(host_mask(p, L), j0, j1, a, b);
  *lo = a;
  *hi = b;
  return ok ? 1 : 0;
}

int attn_host_full_key_tiles(const attn_params* p, int32_t L, int32_t i0, int32_t block_m, int32_t block_n,
                             int32_t* f0, int32_t* f1) {
  if (check_fields(p) != ATTN_OK || !f0 || !f1 || block_m < 1 || block_n < 1 || i0 < 0) return 0;
  int a = 0, b = -1;
  const bool ok = full_key_tiles(host_mask(p, L), i0, block_m, block_n, a, b);
  *f0 = a;
  *f1 = b;
  return ok ? 1 : 0;
}

int attn_host_dkdv_splits(const attn_params* p) {
  if (attn_validate(p) != ATTN_OK) return 0;
  return kv_splits(p);
}

}  // extern "C"
