/*
 * sdpa_attn.h — C ABI of the MI355X (gfx950) fused scaled dot-product attention.
 *
 * The library computes, for every batch b, query head h and query row i,
 *
 *     O[b,i,h,:] = sum_j P_ij V[b,j,kv(h),:],
 *     P_ij = exp(s_ij) / (sum_{j visible} exp(s_ij) + [sink] exp(z_h)),
 *     s_ij = scale * Q[b,i,h,:] . K[b,j,kv(h),:],
 *
 * over visible keys j only, plus the row log-sum-exp, and the backward pass of
 * that function.  Definitions followed:
 *   - score/scale/softmax/attend steps: codelab "Speed up attention on GPU with
 *     cuDNN and TransformerEngine", "How attention works";
 *   - module arguments num_gqa_groups, attn_mask_type, window_size,
 *     scale_factor (default 1/sqrt(head_dim)), separate BSHD Q/K/V with
 *     different Q/K and V head dims, sequence lengths: TransformerEngine
 *     "JAX: Single-GPU Attention with TransformerEngine", sections 1, 2, 4 and
 *     "Other attention knobs";
 *   - softmax_type vanilla / off-by-one / learnable, the softmax_offset
 *     parameter of shape [1, num_heads, 1, 1], the forward outputs (output,
 *     softmax_aux) and the backward outputs (grad_q, grad_k, grad_v,
 *     grad_softmax_offset): PR "[JAX] Add support for sink attention in JAX"
 *     #2225, review summaries and their sequence diagrams.
 *
 * Readings fixed by this ABI (the pages leave them open):
 *   - kv(h) = floor(h / (num_heads / num_gqa_groups)): contiguous head groups;
 *   - window (left, right) is inclusive, i-left <= j <= i+right, -1 unbounded,
 *     intersected with the causal rule j <= i when mask_type is CAUSAL;
 *   - seqlens[b] right-pads queries and keys alike; rows/keys >= seqlens[b]
 *     are invisible;
 *   - off-by-one = an extra logit z = 0; learnable = an extra logit z = alpha_h
 *     (raw value of softmax_offset[h]); z is not multiplied by the scale;
 *   - the LSE output ("softmax_aux") is the natural-log log-sum-exp of each
 *     row including the sink term; empty rows get LSE = -inf (vanilla) or z_h;
 *   - attention dropout, when params.dropout_p > 0, multiplies P_ij in O (and
 *     in the backward) by keep_ij / (1 - p); keep comes from a counter-based
 *     generator keyed by the caller's rng state (see struct attn_params).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers to contiguous row-major arrays; the
 *     library never allocates, never frees and keeps no state between calls.
 *   - Layouts (BSHD): Q, dQ [B,S,Hq,Dqk]; K, dK [B,S,Hkv,Dqk]; V, dV [B,S,Hkv,Dv];
 *     O, dO [B,S,Hq,Dv]; LSE [B,Hq,S] float32; softmax_offset and
 *     d_softmax_offset [Hq] float32; seqlens [B] int32.
 *   - Packed layout (THD), selected by a non-NULL seq_offsets [B+1] int32:
 *     the sequences lie back to back along one token axis, Q, dQ [T,Hq,Dqk];
 *     K, dK [T,Hkv,Dqk]; V, dV [T,Hkv,Dv]; O, dO [T,Hq,Dv] with
 *     T >= seq_offsets[B].  Segment b holds tokens seq_offsets[b] ..
 *     seq_offsets[b+1]-1 (0 = seq_offsets[0] <= seq_offsets[1] <= ..., each
 *     segment at most S = params.seqlen tokens); the first seqlens[b] of them
 *     are valid (all of them when seqlens is NULL) and the rest are padding.
 *     Attention never crosses a segment; positions for the causal and window
 *     rules count from the segment start.  LSE keeps the [B,Hq,S] layout
 *     (row i of segment b).  Tokens at or past seq_offsets[B] are not
 *     touched.  Reading of the TE single-GPU page, section 1, where the
 *     sequence descriptor gives, besides lengths, the start of each packed
 *     sequence and its padding.
 *   - Element type of Q,K,V,O,dO,dQ,dK,dV is params.dtype (bf16 or f32).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = default stream); the
 *     calls return without synchronising.  Inputs are read only.  Outputs are
 *     fully overwritten, padded rows included (O = 0, dQ = dK = dV = 0 there).
 *   - All argument checks run on the host before anything is enqueued; on a
 *     non-zero return nothing was launched, except ATTN_ERR_HIP which reports
 *     a launch failure.
 *   - seqlens and seq_offsets values live on the device and cannot be
 *     checked on the host; kernels clamp lengths and segment sizes to [0, S].
 *     The Python binding checks them.
 */
#ifndef SDPA_ATTN_H
#define SDPA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* params.dtype */
#define ATTN_F32 0
#define ATTN_BF16 1
#define ATTN_FP8 2  /* attn_fwd_fp8 / attn_bwd_fp8 only: E4M3 Q, K, V (E5M2 dO) with descales */
/* 8-bit formats (OCP 8-bit floating point spec) */
#define ATTN_FP8_E4M3 0
#define ATTN_FP8_E5M2 1
/* params.mask_type (codelab section 7; TE single-GPU page section 2) */
#define ATTN_MASK_NONE 0
#define ATTN_MASK_CAUSAL 1
/* params.softmax_type (PR #2225, AttnSoftmaxType) */
#define ATTN_SOFTMAX_VANILLA 0
#define ATTN_SOFTMAX_OFF_BY_ONE 1
#define ATTN_SOFTMAX_LEARNABLE 2

/* status codes */
#define ATTN_OK 0
#define ATTN_ERR_INVALID_ARG (-1)   /* bad size, enum, window, pointer */
#define ATTN_ERR_UNSUPPORTED (-2)   /* valid problem, no kernel: (dtype, Dqk, Dv) or scale < 0 */
#define ATTN_ERR_WORKSPACE (-3)     /* workspace_bytes below the required size */
#define ATTN_ERR_HIP (-4)           /* a HIP launch failed */
#define ATTN_ERR_TOO_LARGE (-5)     /* attn_bwd_noalloc: the problem needs more than its scratch */

/* Problem description.  All fields are plain 32-bit integers or floats for a
 * fixed ABI. */
struct attn_params {
  int32_t batch;          /* B >= 1 */
  int32_t seqlen;         /* S >= 1, shared by queries and keys (self-attention) */
  int32_t num_heads;      /* Hq >= 1 */
  int32_t num_gqa_groups; /* Hkv >= 1, number of K/V heads; Hq % Hkv == 0 */
  int32_t head_dim_qk;    /* Dqk */
  int32_t head_dim_v;     /* Dv */
  int32_t dtype;          /* ATTN_F32 | ATTN_BF16 | ATTN_FP8 (attn_fwd_fp8) */
  int32_t mask_type;      /* ATTN_MASK_NONE | ATTN_MASK_CAUSAL */
  int32_t window_left;    /* >= -1; -1 = unbounded */
  int32_t window_right;   /* >= -1; -1 = unbounded */
  float scale_factor;     /* finite; 0 => 1/sqrt(Dqk); < 0 is ATTN_ERR_UNSUPPORTED */
  int32_t softmax_type;   /* ATTN_SOFTMAX_* */
  /* Attention dropout (TE single-GPU page, "Other attention knobs": a rate
   * and an RNG; PR #2225's forward returns an rng_state).  Reading: inverted
   * dropout on the softmax probabilities, O = (P * Z) V with
   * Z = keep / (1 - t/256), t = round(256 * dropout_p) (the rate is
   * quantised to 1/256; t = 0 disables dropout); the LSE is unchanged.  keep
   * comes from Philox4x32-10 (Salmon et al., SC 2011): one call per 4 x 4
   * block of (query row i, key j) pairs of batch b, query head h, counter
   * (j >> 2, i >> 2, b * num_heads + h, dropout_offset), key (seed_lo,
   * seed_hi); pair (i, j) takes byte (i & 3) * 4 + (j & 3) of the output
   * (word byte / 4, bits 8 * (byte % 4) up) and is kept iff that byte >= t.
   * The (seed, offset) pair is the rng state: pass the same values to the
   * forward and the backward of one step, and advance the offset between
   * steps. */
  float dropout_p;           /* in [0, 1) */
  uint32_t dropout_seed_lo;  /* generator key, low word */
  uint32_t dropout_seed_hi;  /* generator key, high word */
  uint32_t dropout_offset;   /* counter word 3 */
};

/* Host-only check of a problem description; no HIP call.  Returns ATTN_OK,
 * ATTN_ERR_INVALID_ARG or ATTN_ERR_UNSUPPORTED.  Supported (dtype, Dqk, Dv):
 * bf16 with (64,64), (128,128), (192,128); f32 with (64,64). */
int attn_validate(const struct attn_params* p);

/* Workspace bytes the forward / backward call needs (0 if p is invalid).
 * The forward needs none; the backward needs room for the per-row
 * delta = rowsum(dO * O) and LSE * log2(e), the per-block partial sums of
 * d(sink logit), and, for bf16 problems whose dK/dV grid is small (few KV
 * heads, short batches) or whose dK/dV workgroups would walk many rows (long
 * windows, large GQA groups) -- attn_host_dkdv_splits > 1 -- fp32 partial dK
 * and dV of each query-head split of a GQA group.  FP8 problems: the forward
 * needs V transposed per KV head, the backward (attn_bwd_fp8) the per-row
 * terms and K, Q, dO transposed per head (codes). */
size_t attn_fwd_workspace_size(const struct attn_params* p);
size_t attn_bwd_workspace_size(const struct attn_params* p);

/* Workspace bytes with which attn_bwd also keeps the backward's dS matrix
 * (codelab "Speed up attention on GPU with cuDNN and TransformerEngine",
 * "How attention works": the score gradient that dK = scale dS^T Q and
 * dQ = scale dS K share) and computes dQ from it instead of recomputing
 * S = QK^T and dP = dO V^T a second time (with dropout the stored dS has the
 * dropout applied, so dQ needs no random bytes); 0 when the problem has no
 * such path (fp32, FP8, or more than 2^31 - 1 blocks per head: sequences of
 * millions of tokens without a window) or p is invalid.  The extra room is
 * B * Hq * n * 8 KiB: dS in bf16 blocks of 32 rows x 128 keys, n the number
 * of blocks over all 128-key tiles of the rows that see each tile (in 64-row
 * steps, at the full length S): about S^2 / 4096 without a mask, half that
 * causal, S (window + 192) / 4096 with a window (1.1 GB for B=4, S=4096,
 * Hq=32 and a 1024-key causal window; 4.4 GB for B=2, S=4096, Hq=128,
 * causal).  attn_bwd takes this path whenever workspace_bytes is at least
 * this size (and > 0), and so do attn_bwd_stage (stage order 1, 3, 2, 4
 * then) and attn_bwd_bias (dBias then summed from the stored blocks);
 * attn_bwd_noalloc never does.  Results agree with the recomputing path to
 * rounding (dS is the same bf16 value either way; S, dP and delta are summed
 * in another order, and a shared bias's gradient sums the bf16 dS blocks
 * where the other path sums fp32 dS), and are bitwise reproducible run to
 * run on either path. */
size_t attn_bwd_ds_workspace_size(const struct attn_params* p);

/* Forward.  Writes O [B,S,Hq,Dv] (packed: [T,Hq,Dv]) and LSE [B,Hq,S].
 *   softmax_offset: [Hq] float32 sink logits; required for LEARNABLE,
 *                   ignored otherwise (may be NULL).
 *   seqlens:        [B] int32 valid lengths, or NULL for all S (packed: the
 *                   whole segment).
 *   seq_offsets:    [B+1] int32 segment starts of packed (THD) tensors, or
 *                   NULL for BSHD.
 *   workspace:      may be NULL when workspace_bytes >= attn_fwd_workspace_size. */
int attn_fwd(const struct attn_params* p, const void* q, const void* k, const void* v,
             const float* softmax_offset, const int32_t* seqlens, const int32_t* seq_offsets,
             void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* Backward of the forward above for upstream gradient d_o (PR #2225 backward:
 * grad_q, grad_k, grad_v, grad_softmax_offset).  o and lse must be the
 * forward's outputs for the same inputs.  Writes dQ, dK, dV.
 *   d_softmax_offset: [Hq] float32, overwritten with d(loss)/d(z_h) summed
 *     over batches and rows.  Required for LEARNABLE; optional for OFF_BY_ONE
 *     (gradient w.r.t. the implicit zero logit); must be NULL for VANILLA.
 *   workspace: at least attn_bwd_workspace_size(p) bytes, 256-byte aligned;
 *     with attn_bwd_ds_workspace_size(p) bytes or more (when that is > 0)
 *     dQ comes from the stored dS (see there).
 *   seqlens, seq_offsets: as for attn_fwd, and the same values.
 * dK/dV accumulate the query heads of a GQA group in a fixed order, and dQ and
 * d_softmax_offset are reduced in a fixed order: results are bitwise
 * reproducible run to run. */
int attn_bwd(const struct attn_params* p, const void* q, const void* k, const void* v,
             const void* o, const void* d_o, const float* lse, const float* softmax_offset,
             const int32_t* seqlens, const int32_t* seq_offsets, void* dq, void* dk, void* dv,
             float* d_softmax_offset, void* workspace, size_t workspace_bytes, void* stream);

/* One stage of attn_bwd, same arguments and checks as attn_bwd.  attn_bwd
 * runs the stages 1..4 in order on one stream, or 1, 3, 2, 4 when the
 * workspace holds the stored dS (at least attn_bwd_ds_workspace_size bytes:
 * stage 1 is then the pre-pass for bf16 too, stage 3 stores dS and stage 2
 * computes dQ from it); each stage needs the ones before it in that order
 * (stage 4 needs only stages 1 and 2 on the recomputing path, stage 1 on the
 * other).
 *   1 ATTN_BWD_STAGE_PREPROCESS  delta = rowsum(dO * O), LSE * log2(e) and
 *                                per-block partials of the sink gradient
 *                                (fp32; for bf16 stage 2 does this work and
 *                                stage 1 launches nothing)
 *   2 ATTN_BWD_STAGE_DQ          dQ
 *   3 ATTN_BWD_STAGE_DKDV        dK, dV
 *   4 ATTN_BWD_STAGE_OFFSET_GRAD d_softmax_offset (no-op when it is NULL)
 * Any other stage value returns ATTN_ERR_INVALID_ARG. */
#define ATTN_BWD_STAGE_PREPROCESS 1
#define ATTN_BWD_STAGE_DQ 2
#define ATTN_BWD_STAGE_DKDV 3
#define ATTN_BWD_STAGE_OFFSET_GRAD 4
int attn_bwd_stage(int stage, const struct attn_params* p, const void* q, const void* k, const void* v,
                   const void* o, const void* d_o, const float* lse, const float* softmax_offset,
                   const int32_t* seqlens, const int32_t* seq_offsets, void* dq, void* dk, void* dv,
                   float* d_softmax_offset, void* workspace, size_t workspace_bytes, void* stream);

/* Attention with an additive bias.  TE single-GPU page, "Other attention
 * knobs": the module takes a bias tensor with a bias type; PR #2225's backward
 * returns grad_bias next to grad_q, grad_k, grad_v.  Neither gives the formula
 * or the shapes; reading: a post-scale bias added to the scores of visible
 * pairs,
 *     s_ij = scale * Q[b,i,h,:] . K[b,j,kv(h),:] + bias[b', h', i, j],
 * with bias [bias_batch, bias_heads, S, S] in params.dtype, bias_batch in
 * {1, B} and bias_heads in {1, Hq} (a size-1 dim is shared: b' = 0 or b,
 * h' = 0 or h).  Rows and keys are positions within the sequence (within
 * the segment for packed inputs).  Masked pairs ignore the bias.
 * Supported: bf16 with (Dqk, Dv) = (64, 64) or (128, 128), S a multiple of
 * 8 and S <= 46336 (one bias matrix within 4 GiB); anything else with a bias
 * is ATTN_ERR_UNSUPPORTED (pad S and pass seqlens for other lengths).  bias
 * and d_bias must be 16-byte aligned (else ATTN_ERR_INVALID_ARG).  Otherwise
 * as attn_fwd / attn_bwd (same checks, layouts, stream and ownership rules). */
int attn_fwd_bias(const struct attn_params* p, const void* q, const void* k, const void* v,
                  const void* bias, int32_t bias_batch, int32_t bias_heads,
                  const float* softmax_offset, const int32_t* seqlens, const int32_t* seq_offsets,
                  void* o, float* lse, void* workspace, size_t workspace_bytes, void* stream);
/* Backward with the same bias.  d_bias: NULL (not computed) or a device
 * array of the bias's shape, overwritten with d(loss)/d(bias): dS = P * (dP -
 * delta) on the pairs each sharing (batch, head) sees, zero elsewhere,
 * summed over the batches and heads that share a bias matrix in ascending
 * order (bitwise reproducible).  With attn_bwd_ds_workspace_size(p) bytes of
 * workspace or more (no dropout) the dK/dV kernel stores dS and dQ and dBias
 * are computed from it, which for a bias shared over batches or heads saves
 * recomputing S and dP once per sharing (batch, head) pair. */
int attn_bwd_bias(const struct attn_params* p, const void* q, const void* k, const void* v,
                  const void* o, const void* d_o, const float* lse, const void* bias,
                  int32_t bias_batch, int32_t bias_heads, void* d_bias, const float* softmax_offset,
                  const int32_t* seqlens, const int32_t* seq_offsets, void* dq, void* dk, void* dv,
                  float* d_softmax_offset, void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free backward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments, checks, kernels and results as attn_bwd, minus
 * the workspace: the backward runs in a scratch array of
 * ATTN_NOALLOC_SCRATCH_BYTES that the library holds in device memory on each
 * GPU it runs on, from the first call on that GPU until the process ends.
 * Nothing is allocated or freed per call (no hipMalloc, hipFree or
 * allocating library routine).
 *   - A problem whose attn_bwd_workspace_size exceeds the scratch returns
 *     ATTN_ERR_TOO_LARGE before anything is enqueued; use attn_bwd then.
 *   - Work is enqueued on `stream`, which must belong to the current device
 *     (the scratch used is the current device's).
 *   - Every call on one GPU shares that GPU's scratch: calls that overlap on
 *     one GPU (other streams, other threads, without ordering between them)
 *     race and give wrong results.  Calls on one stream are ordered.  Every
 *     value a call reads from the scratch it has written first, so nothing
 *     needs clearing between calls. */
#define ATTN_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)
int attn_bwd_noalloc(const struct attn_params* p, const void* q, const void* k, const void* v,
                     const void* o, const void* d_o, const float* lse, const float* softmax_offset,
                     const int32_t* seqlens, const int32_t* seq_offsets, void* dq, void* dk, void* dv,
                     float* d_softmax_offset, void* stream);

/* ---- FP8 (codelab "Speed up attention on GPU with cuDNN and
 * TransformerEngine", section 10: attention under FP8 autocast with a
 * DelayedScaling recipe, HYBRID format = E4M3 forward / E5M2 backward tensors,
 * an amax history and the "max" rule).  The page fixes neither the formats'
 * encodings nor the arithmetic; readings:
 *   - formats E4M3 and E5M2 of the OCP 8-bit floating point spec, encoded by
 *     round-to-nearest-even with saturation to the largest finite value;
 *   - per-tensor scaling: codes = encode(x * scale), value = code * descale;
 *   - the forward quantizes P relative to the exact row max,
 *     P8 = E4M3(256 exp(s - m_i)), and normalises by the unquantized sum:
 *     O_i = descale_v / (256 l_i) sum_j P8_ij V8_j;
 *   - the backward (HYBRID: dO arrives as E5M2 codes) recomputes
 *     P = exp(s - LSE), delta_i = dO_i . O_i, dP = dO V^T, dS = P (dP - delta)
 *     in fp32 and feeds FP8 operands to the gradient products:
 *     dV = sum_i E4M3(256 P_ij) / 256 dO_i, and with a per-tensor dS scale
 *     s_ds (the recipe's delayed scale; the call returns this step's amax of
 *     dS) dK = scale / s_ds sum_i E5M2(s_ds dS_ij) Q_i,
 *     dQ = scale / s_ds sum_j E5M2(s_ds dS_ij) K_j.
 * Built: forward, backward, the quantization with amax and the
 * delayed-scaling scale update.  attn_fwd / attn_bwd with ATTN_FP8 return
 * ATTN_ERR_UNSUPPORTED (use the entry points below). */

/* FP8 forward.  p->dtype = ATTN_FP8; Dqk = Dv in {64, 128}; dropout_p = 0.
 * q, k, v: E4M3 codes (1 byte each) in the layouts of attn_fwd, 16-byte
 * aligned.  descale_qkv: device float[3] = the descales of q, k, v (kept on
 * the device so a recipe can update them without a host round trip).  o:
 * bf16 [B,S,Hq,Dv] (packed: [T,Hq,Dv]); lse: float32 [B,Hq,S] (natural log,
 * sink included).  workspace: attn_fwd_workspace_size(p) bytes, 256-byte
 * aligned (V transposed per KV head).  Other arguments as attn_fwd. */
int attn_fwd_fp8(const struct attn_params* p, const void* q, const void* k, const void* v,
                 const float* descale_qkv, const float* softmax_offset, const int32_t* seqlens,
                 const int32_t* seq_offsets, void* o, float* lse, void* workspace,
                 size_t workspace_bytes, void* stream);

/* FP8 backward.  p as attn_fwd_fp8.  q, k, v: the forward's E4M3 codes; o:
 * the forward's bf16 output; d_o: E5M2 codes of dO ([B,S,Hq,Dv] / [T,Hq,Dv]);
 * all 16-byte aligned.  lse: the forward's [B,Hq,S].  descale_qkvdo: device
 * float[4], the descales of q, k, v, d_o.  ds_scale: device float[1], the
 * scale of dS before its E5M2 encoding.  amax_ds: device float[1], receives
 * max |dS| over the visible pairs (overwritten).  dq, dk, dv: bf16 outputs in
 * the layouts of q, k, v (padded rows and keys written as zeros).
 * d_softmax_offset as attn_bwd.  workspace: attn_bwd_workspace_size(p) bytes,
 * 256-byte aligned (delta, LSE log2 e, sink partials, and K, Q, dO transposed
 * per head).  Deterministic: no atomics on the gradients. */
int attn_bwd_fp8(const struct attn_params* p, const void* q, const void* k, const void* v, const void* o,
                 const void* d_o, const float* lse, const float* descale_qkvdo, const float* ds_scale,
                 float* amax_ds, const float* softmax_offset, const int32_t* seqlens,
                 const int32_t* seq_offsets, void* dq, void* dk, void* dv, float* d_softmax_offset,
                 void* workspace, size_t workspace_bytes, void* stream);

/* Per-tensor quantization: out[i] = encode(clamp(x[i] * scale[0], -max,
 * max)) in format fmt (ATTN_FP8_E4M3 / ATTN_FP8_E5M2), and amax[0] = max |x|
 * (NaN elements excluded).  x: n elements of x_dtype (ATTN_F32 32-byte or
 * ATTN_BF16 16-byte aligned); out: n bytes, 8-byte aligned; scale, amax:
 * device float[1].  All on `stream`; amax is overwritten. */
int attn_fp8_quantize(const void* x, int32_t x_dtype, size_t n, int32_t fmt, const float* scale,
                      uint8_t* out, float* amax, void* stream);

/* One delayed-scaling step, on the device: amax_history[0 .. history_len)
 * (1 <= history_len <= 4096, newest first) becomes {amax[0], previous
 * history without its oldest entry}; then scale[0] = fmt_max / max(history) /
 * 2^margin when that max is positive and finite (else scale[0] is kept), and
 * descale[0] = 1 / scale[0]. */
int attn_fp8_update_scale(float* amax_history, int32_t history_len, const float* amax, int32_t fmt,
                          int32_t margin, float* scale, float* descale, void* stream);

/* Static text for a status code. */
const char* attn_status_string(int status);

/* Tile sizes (query rows x keys) the forward kernel uses for problem p.
 * Returns ATTN_OK or the attn_validate error. */
int attn_fwd_tile_shape(const struct attn_params* p, int32_t* block_m, int32_t* block_n);

/* ---- mask engine exports (test and inspection) --------------------------
 * Tile classes: 0 = SKIP (no visible pair), 1 = PARTIAL (per-element
 * predicate), 2 = FULL (every pair visible).  The device variants run the
 * same integer code the kernels run. */

/* Device: out[b][qt][kt] (int8, device, B * ceil(S/block_m) * ceil(S/block_n)
 * entries) = class of query tile qt x key tile kt for batch b. */
int attn_debug_tile_map(const struct attn_params* p, const int32_t* seqlens, int32_t block_m,
                        int32_t block_n, int8_t* out, void* stream);

/* Device: out[b][i][j] (uint8, device, B*S*S entries) = 1 iff query i sees key j. */
int attn_debug_mask_probe(const struct attn_params* p, const int32_t* seqlens, uint8_t* out,
                          void* stream);

/* Device: out[b][h][i][j] (uint8, device, B*Hq*S*S entries) = 1 iff pair
 * (i, j) of batch b, query head h is kept by dropout (every pair, visible or
 * not), from the same device generator the kernels use. */
int attn_debug_dropout_mask(const struct attn_params* p, uint8_t* out, void* stream);

/* Host: same tile map from host seqlens (NULL = all S) into host memory. */
int attn_host_tile_map(const struct attn_params* p, const int32_t* seqlens, int32_t block_m,
                       int32_t block_n, int8_t* out);

/* Host: contiguous range [*lo, *hi] of keys visible from any of the query
 * rows i0..i1 (inclusive), for valid length L; returns 1 if non-empty, else 0. */
int attn_host_key_range(const struct attn_params* p, int32_t L, int32_t i0, int32_t i1,
                        int32_t* lo, int32_t* hi);

/* Host: contiguous range [*lo, *hi] of query rows that see any of the keys
 * j0..j1 (inclusive); returns 1 if non-empty, else 0. */
int attn_host_query_range(const struct attn_params* p, int32_t L, int32_t j0, int32_t j1,
                          int32_t* lo, int32_t* hi);

/* Host: number of query-head splits of a GQA group the bf16 dK/dV stage
 * uses for this problem (1 = none; 0 if p is invalid): the smallest divisor
 * s of G for which ceil(S/128)*B*Hkv*s >= 1024 and one workgroup walks at
 * most 512 blocks of 32 query rows over its G/s heads (else G), lowered to
 * the largest divisor whose fp32 partials take at most 1 GiB.  With s > 1 splits,
 * s workgroups per (128-key tile, batch, KV head) each walk G/s of the
 * group's query heads and write fp32 partials, which a second kernel adds in
 * split order, so dK and dV stay bitwise reproducible. */
int attn_host_dkdv_splits(const struct attn_params* p);

/* Host: key tiles [*f0, *f1] (tile t = keys t*block_n .. t*block_n+block_n-1)
 * that every query row i0 .. i0+block_m-1 sees in full, for valid length L:
 * the tiles attn_host_tile_map marks 2 for that row block.  Returns 1 if
 * there are any, else 0 (also on invalid arguments). */
int attn_host_full_key_tiles(const struct attn_params* p, int32_t L, int32_t i0, int32_t block_m,
                             int32_t block_n, int32_t* f0, int32_t* f1);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_ATTN_H */
