// Backward attention, dK and dV, bf16 inputs, fp32 accumulation, gfx950 MFMA 32x32x16.
// Built without the VGPR-form MFMA option: dK and dV (and the S / dP blocks in
// flight) accumulate in AGPRs, leaving the VGPRs for operands and softmax work.
//
// With P = exp(scale * Q K^T - LSE) recomputed from the forward's LSE and
// delta_i = rowsum(dO * O) from the pre-pass (PR #2225 backward: dz = dO in,
// grad_q, grad_k, grad_v out):
//     dP = dO V^T,  dS = P * (dP - delta),
//     dV = P^T dO,  dK = scale * dS^T Q,  dQ = scale * dS K.
// This kernel (deterministic, no atomics): a workgroup owns BN = 128 keys of
// one (batch, KV head); each wave owns 32 keys and keeps dK, dV in registers
// while the workgroup walks the G query heads of the group in ascending order
// and, for each, the visible query rows in ascending order, 32 rows (one
// block) at a time; the GQA sum is therefore a fixed-order register
// accumulation.  When the grid of key tiles would be too small to fill the
// GPU (few KV heads, short batches), the G heads are split over n_splits
// workgroups; each writes fp32 partial dK, dV and a second kernel adds the
// partials in split order.  dQ has its own kernel.
//
// Software pipeline.  Per block u a wave runs three dependent phases:
//   A(u): S = Q K^T and dP = dO V^T for its 32 keys          (MFMA)
//   B(u): P = exp2(S c - lse2), masked; dS = P (dP - delta)   (VALU)
//   C(u): dV^T += dO^T P,  dK^T += Q^T dS                     (MFMA)
// Iteration u issues A(u+1), B(u) and C(u-1): three independent groups in
// one basic block, so the scheduler can fill the MFMA pipe with A and C
// while B's exp / FMA work issues in between (one wave per SIMD has no other
// wave to hide its softmax behind).  S/dP and P/dS each alternate between two
// register sets.  An iteration runs in four chunks whose LDS operands are read
// one chunk ahead, the first chunk's during the last chunk of the iteration
// before (A's only where no barrier lies in between).
//
// Query rows are staged 64 at a time (two blocks) in a ring of three LDS
// buffers filled by direct memory-to-LDS copies: Q and dO tiles (swizzled
// rows) plus the rows' lse2 and delta.  Iteration u touches the stages of
// blocks u-1, u, u+1, so the copy of stage s+1 is issued after the barrier
// that opens stage s (at iteration 2s-1), when stage s-2 is no longer read,
// and has two iterations to land.  The loop is unrolled over the six phases
// of (block parity, ring slot) so every register set and LDS offset is a
// compile-time constant.
//
// Masks: every wave evaluates the visibility predicate per element (two
// integer compares against the rows that see its key), on every block.  The
// workgroup's blocks are computed by all four waves, also where a wave's own
// keys see none of a block's rows (its P is then zero).
//
// MFMA operand layouts: a lane of a 32x32 accumulator owns one column and 16
// rows (acc_row).  Contractions over head dims read 16-byte row pieces of a
// swizzled row-major LDS tile (RowReads); contractions over the sequence take
// the accumulator-side operand straight from registers and the other one
// with LDS transpose loads from the same tile (TrReads).
//
// DROP (attention dropout, dropout.h): with Z = keep / (1 - p), dV = (P Z)^T
// dO and dS = P (Z dP - delta).  B keeps P * keep for dV (the 1 / (1 - p)
// factor is applied once, to dV at the end) and P (Z dP - delta) for dK; the
// random bytes of a lane's key and one 4-row group come from one generator
// call, which is exactly one pipeline chunk's share of B.
//
// DSOUT (the stored-dS backward): the kernel also writes each block's bf16 dS
// (the B operand of its dK products) to the workspace, block by block, for a
// dQ kernel that contracts it with K instead of recomputing S and dP
// (attn_bwd_dq_ds_bf16.hip) and, with a bias, for the dBias sum
// (dbias_from_ds_kernel); layout and store rules at the stores below.
//
// BIAS (additive post-scale attention bias, P = exp(scale q.k + bias - LSE)):
// each stage also holds the bias tile of its 64 rows x the workgroup's 128
// keys (swizzled rows, copied with Q and dO).  A lane needs its key's values
// for the rows of its accumulator elements; one LDS transpose load hands it
// the four rows of one B chunk, in accumulator order (TrReads).
#include <type_traits>

#include "dropout.h"
#include "launch.h"

// Issue pattern inside a pipeline chunk (build-time overridable for tuning
// sweeps): LDS reads and VALU instructions placed after each MFMA.
#ifndef SDPA_DKDV_DS
#define SDPA_DKDV_DS 2
#endif
#ifndef SDPA_DKDV_VALU
#define SDPA_DKDV_VALU 2
#endif

namespace sdpa {

template <int V>
using IC = std::integral_constant<int, V>;

template <int DQK, int DV, bool BIAS>
struct DkdvCfg {
  static constexpr int BN = 128;  // keys per workgroup (32 per wave)
  static constexpr int BMQ = 64;  // query rows per stage (two 32-row blocks)
  static constexpr int NBUF = 3;  // stages resident in LDS
  static constexpr int NT = 256;
  static constexpr int QCH = DQK / 8, OCH = DV / 8;    // 16-byte chunks per row
  static constexpr int QT = BMQ * DQK, OT = BMQ * DV;  // elements per tile
  static constexpr int BT = BIAS ? BMQ * BN : 0;       // bias tile [BMQ][BN]
  static constexpr int STAGE = QT + OT + BT;  // tiles of a ring slot: Q, dO, bias
  static constexpr int RT = 2 * BMQ * 2;      // row terms of a ring slot: lse2 and delta (f32)
  static constexpr int LDS_ELEMS = NBUF * (STAGE + RT);
};

template <int DQK, int DV, bool DROP, bool BIAS, bool DSOUT>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_kernel(KArgs a) {
  using C = DkdvCfg<DQK, DV, BIAS>;
  // Without dropout, delta is folded into the dP products: their
  // accumulator starts at delta and V enters negated, so it ends at
  // delta - dP and P times it is -dS with no subtraction; dK then
  // accumulates -dK, negated at the end (all exact sign changes).
  constexpr bool FOLD = !DROP;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  // Ring slot `buf`: tiles Q [BMQ][DQK], dO [BMQ][DV], bias [BMQ][BN]
  // (swizzled) at buf * STAGE; after the NBUF slots' tiles, its row terms
  // lse2 [BMQ] and delta [BMQ].
  auto qtile = [&](int buf) __attribute__((always_inline)) { return lds + buf * C::STAGE; };
  auto otile = [&](int buf) __attribute__((always_inline)) { return lds + buf * C::STAGE + C::QT; };
  auto btile = [&](int buf) __attribute__((always_inline)) { return lds + buf * C::STAGE + C::QT + C::OT; };
  auto lse_s = [&](int buf) __attribute__((always_inline)) { return reinterpret_cast<float*>(lds + C::NBUF * C::STAGE + buf * C::RT); };
  auto delta_s = [&](int buf) __attribute__((always_inline)) { return lse_s(buf) + C::BMQ; };

  const int tid = threadIdx.x, w = wave_id(tid), lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  // Workgroup id -> (batch, kv head, head split; key tile).  Grouped order:
  // the key tiles of one (batch, kv head, split) read overlapping Q / dO
  // rows, so they run together on one XCD (xcd_group_item) and the rows a
  // tile copies are still in that XCD's L2 when its neighbours reach them.
  // Otherwise consecutive ids cover all groups of one key tile (with
  // B*Hkv*n_splits a multiple of 8 a group always lands on the same XCD).
  // Key tiles in ascending order: under a causal mask the first ones see the
  // most queries.  Head split hs of n_splits covers query heads
  // hs*Gs .. hs*Gs+Gs-1 of the group.
  const int nsp = a.n_splits, Gs = a.G / nsp;
  int r, kt;
  if constexpr (kGroupedOrder<DQK>) {
    xcd_group_item(blockIdx.x, a.B * a.Hkv * nsp, (a.S + C::BN - 1) / C::BN, r, kt);
  } else {
    kt = blockIdx.x / (a.B * a.Hkv * nsp);
    r = blockIdx.x % (a.B * a.Hkv * nsp);
  }
  kt = __builtin_amdgcn_readfirstlane(kt);  // wave-uniform: scalar registers
  r = __builtin_amdgcn_readfirstlane(r);
  const int hs = r % nsp;
  r /= nsp;
  const int b = r / a.Hkv, g = r % a.Hkv;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  const DropGen dg = drop_gen(a);
  const int j0 = kt * C::BN;
  const int kj = j0 + w * 32 + l32;
  int qlo_k, qhi_k;  // rows that see this lane's key
  col_query_bounds(m, kj, qlo_k, qhi_k);
  // Rows that see all 32 keys of this wave: both bounds grow with the key,
  // so they run from the last key's first row to the first key's last row
  // (none if the wave holds keys past the valid length).  Blocks of such
  // rows need no mask.
  int all_lo, all_hi;
  {
    const int kw0 = j0 + w * 32;
    int lo_a, hi_a, lo_b, hi_b;
    col_query_bounds(m, kw0 + 31, lo_a, hi_a);
    col_query_bounds(m, kw0, lo_b, hi_b);
    all_lo = lo_a;
    all_hi = hi_b;
    if (kw0 + 31 >= m.L) { all_lo = 1; all_hi = 0; }
  }

  // K^T / V^T operands: lane holds key kj, dims [ks*16 + hf*8, +8); buffer
  // resources end at the valid length, so keys >= L read as zeros.
  bf16x8 kreg[DQK / 16], vreg[DV / 16];
  {
    const size_t kstride = (size_t)a.Hkv * DQK, vstride = (size_t)a.Hkv * DV;
    const __amdgpu_buffer_rsrc_t kres = buf_rsrc(static_cast<const uint16_t*>(a.k) + (seq_row0(a, b) * a.Hkv + g) * DQK,
                                                 (uint32_t)(m.L * kstride * 2));
    const __amdgpu_buffer_rsrc_t vres = buf_rsrc(static_cast<const uint16_t*>(a.v) + (seq_row0(a, b) * a.Hkv + g) * DV,
                                                 (uint32_t)(m.L * vstride * 2));
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks)
      kreg[ks] = as_bf16x8(buf_load16(kres, (uint32_t)(kj * kstride + ks * 16 + hf * 8) * 2));
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks) {
      u32x4 vw = buf_load16(vres, (uint32_t)(kj * vstride + ks * 16 + hf * 8) * 2);
      if constexpr (FOLD) vw ^= 0x80008000u;  // -V, exact
      vreg[ks] = as_bf16x8(vw);
    }
  }
  f32x16 dk[DQK / 32], dv[DV / 32];
#pragma unroll
  for (int i = 0; i < DQK / 32; ++i) dk[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < DV / 32; ++i) dv[i] = f32x16{};

  // Stages: (head of the group, 64-row step) pairs in ascending order.
  int qlo = 0, qhi = -1;
  if (!query_range(m, j0, j0 + C::BN - 1, qlo, qhi)) { qlo = 0; qhi = -1; }
  const int qs0 = qlo / C::BMQ;
  const int nsteps = qhi < 0 ? 0 : qhi / C::BMQ - qs0 + 1;
  const int T = nsteps * Gs;   // stages
  const int NB = 2 * T;        // 32-row blocks
  const int NI = NB > 0 ? (NB + 4) / 6 * 6 : 0;  // pipeline iterations after the first (multiple of 6, >= NB-1)
  const int TP = ((NI + 1) >> 1) + 1;            // stages touched, the padding ones included
  // Walk over the stages in order, kept incrementally (no divisions in the
  // loop): head offset within the group and first row.  Padding stages
  // start at row S: their copies read nothing and land zeros.
  struct StageWalk {
    int t, hh, q0;
  };
  const int q_first = qs0 * C::BMQ, q_last = (qs0 + nsteps - 1) * C::BMQ;
  auto walk_next = [&](StageWalk& st) __attribute__((always_inline)) {
    ++st.t;
    st.q0 += C::BMQ;
    if (st.q0 > q_last) {
      st.q0 = q_first;
      ++st.hh;
    }
    if (st.t >= T) {
      st.q0 = a.S;
      st.hh = 0;
    }
  };

  const uint16_t* Qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* dOg = static_cast<const uint16_t*>(a.d_o);
  const size_t qstride = (size_t)a.Hq * DQK, ostride = (size_t)a.Hq * DV;
  const size_t row0 = seq_row0(a, b);
  const TileCopy<C::BMQ, C::QCH, C::NT> qcopy(tid, (uint32_t)(qstride * 2));
  const TileCopy<C::BMQ, C::OCH, C::NT> ocopy(tid, (uint32_t)(ostride * 2));
  const RowReads<C::QCH> qrd(lane);
  const RowReads<C::OCH> ord(lane);
  const TrReads<C::QCH> qtr(lane);
  const TrReads<C::OCH> otr(lane);
  // A DS instruction's immediate offset has 16 bits.  Tiles that start at
  // 64 KiB or beyond are read through copies of the per-lane offsets that
  // already hold the 64 KiB, and the row terms through one per-lane base;
  // both are opaque to the compiler, so they stay in registers instead of
  // being rebuilt with an add before every read.  (Not in the 192-dim
  // dropout variant, whose registers are full: there the compiler adds.)
  constexpr int kFar = 65536;  // bytes
  constexpr bool FAR = !(DROP && DQK > 128);
  auto opaque = [](uint32_t& x) __attribute__((always_inline)) { asm volatile("" : "+v"(x)); };
  RowReads<C::QCH> qrd_f = qrd;
  TrReads<C::QCH> qtr_f = qtr;
  RowReads<C::OCH> ord_f = ord;
  TrReads<C::OCH> otr_f = otr;
  if constexpr (FAR) {
#pragma unroll
    for (int i = 0; i < C::QCH / 2; ++i) { qrd_f.off[i] += kFar; opaque(qrd_f.off[i]); }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < C::QCH / 4; ++i) { qtr_f.off[h][i] += kFar; opaque(qtr_f.off[h][i]); }
  }
  if constexpr (FAR && C::OCH == C::QCH) {
    ord_f = qrd_f;  // same offsets: share the registers
    otr_f = qtr_f;
  } else if constexpr (FAR) {
#pragma unroll
    for (int i = 0; i < C::OCH / 2; ++i) { ord_f.off[i] += kFar; opaque(ord_f.off[i]); }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < C::OCH / 4; ++i) { otr_f.off[h][i] += kFar; opaque(otr_f.off[h][i]); }
  }
  // Row reads / transpose reads of the tile at element offset O (a constant).
  auto rows_at = [&](auto oc, const auto& near, const auto& far, int rb, int ks) __attribute__((always_inline)) {
    constexpr int O = decltype(oc)::value;
    if constexpr (FAR && 2 * O >= kFar) return far.read(lds + O - kFar / 2, rb, ks);
    else return near.read(lds + O, rb, ks);
  };
  auto tr_at = [&](auto oc, const auto& near, const auto& far, int pos0, int db) __attribute__((always_inline)) {
    constexpr int O = decltype(oc)::value;
    if constexpr (FAR && 2 * O >= kFar) return far.read(lds + O - kFar / 2, pos0, db);
    else return near.read(lds + O, pos0, db);
  };
  // lse2 (term 0) or delta (term 1) of rows r .. r+3 of ring slot buf, r a
  // constant plus hf * 4 (the lane half's share).
  uint32_t rt_lane = (uint32_t)(C::NBUF * C::STAGE * 2 + hf * 16);
  if constexpr (FAR) opaque(rt_lane);
  auto rterm = [&](int buf, int term, int r) __attribute__((always_inline)) {
    return *reinterpret_cast<const f32x4*>(reinterpret_cast<const char*>(lds) + rt_lane +
                                           (buf * C::RT * 2 + term * C::BMQ * 4 + r * 4));
  };
  const TileCopy<C::BMQ, C::BN / 8, C::NT> bcopy(tid, (uint32_t)a.S * 2);
  const TrReads<C::BN / 8> btr(lane);
  auto issue_stage = [&](const StageWalk& st, int buf) __attribute__((always_inline)) {
    const int h = g * a.G + hs * Gs + st.hh;
    const int q0 = st.q0;
    qcopy.issue(Qg + (row0 * a.Hq + h) * DQK, (uint32_t)(qstride * 2), q0, m.L, qtile(buf));
    ocopy.issue(dOg + (row0 * a.Hq + h) * DV, (uint32_t)(ostride * 2), q0, m.L, otile(buf));
    if constexpr (BIAS) {
      // Bias rows q0 .. q0+63, keys j0 .. j0+127 of head h: the resource ends
      // where row L starts, so rows past the valid length (and keys past S
      // on the last valid row) arrive as zeros and nothing past the [S, S]
      // matrix is read; keys past S on earlier rows read the next row (pairs
      // the mask hides).
      const long long left = (long long)(m.L - q0) * a.S - j0;
      bcopy.issue_bytes(bias_matrix(a, b, h) + (size_t)q0 * a.S + j0, left > 0 ? (uint32_t)(left * 2) : 0u,
                        btile(buf));
    }
    // lse2 (wave 0) and delta (wave 1) of rows q0 .. q0+63, one 4-byte copy
    // per lane; rows past S arrive as zeros.
    if (w < 2) {
      const float* src = (w == 0 ? a.lse2 : a.delta) + ((size_t)b * a.Hq + h) * a.S;
      float* dst = w == 0 ? lse_s(buf) : delta_s(buf);
      lds_dma4(buf_desc(src, (uint32_t)a.S * 4), lds_addr(dst), (uint32_t)(q0 + lane) * 4);
    }
  };

  const float c = a.scale_log2;
  // delta of rows rb + acc_row(i, hf) of a stage: the dP accumulator's start.
  auto delta_init = [&](int buf, int rb) __attribute__((always_inline)) {
    f32x16 r;
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const f32x4 d = rterm(buf, 1, rb + ig * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) r[ig * 4 + e] = d[e];
    }
    return r;
  };
  f32x16 S[2], DP[2];        // S / dP of the block in B and of the one in A
  u32x4 PW[2][2], DW[2][2];  // bf16 P / dS pairs: B operands of the block's two 16-row K-steps

  // A(u): S and dP of block u (rows rb .. rb+31 of a ring slot).
  auto phase_a = [&](const uint16_t* Qs, const uint16_t* Os, int rb, f32x16& s, f32x16& dp) __attribute__((always_inline)) {
    s = f32x16{};
    dp = FOLD ? delta_init(0, rb) : f32x16{};
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks) s = mfma32(as_bf16x8(qrd.read(Qs, rb, ks)), kreg[ks], s);
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks) dp = mfma32(as_bf16x8(ord.read(Os, rb, ks)), vreg[ks], dp);
  };
  // B(u): element i of the accumulators is query row qrow0 + acc_row(i, hf),
  // key kj; lse2 / delta come from the stage at offset rb.
  // Dropout bytes of key kj and rows q0 + g*8 + hf*4 + 0..3, g = 0..3 (the
  // accumulator elements 4g .. 4g+3 of a block starting at row q0): one
  // generator call per lane, shared across the lane quad.
  auto drop_rows = [&](int bh, int q0, uint32_t(&rnd4)[4]) __attribute__((always_inline)) {
    drop_cols_quad(dg, bh, q0 + hf * 4, kj, rnd4);
  };
  // Bias of rows rb + k*8 + hf*4 + 0..3 (B chunk k of the block at rb) for
  // this lane's key: the k%2 half of the transpose read at rb + (k/2)*16.
  auto bias_chunk = [&](const uint16_t* bt, int rb, int k) __attribute__((always_inline)) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const char* t = reinterpret_cast<const char*>(bt) + (rb + (k >> 1) * 16) * (C::BN / 8) * 16;
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + btr.off[k & 1][w])));
  };
  // Score of element e of a B chunk with its bias added (unscaled units).
  auto biased = [&](float sv, const u32x2& bw, int e) __attribute__((always_inline)) {
    if constexpr (BIAS) {
      const uint32_t word = bw[e >> 1];
      return fmaf((e & 1) ? bf16_hi(word) : bf16_lo(word), a.inv_scale, sv);
    } else {
      return sv;
    }
  };
  auto phase_b = [&](int buf, const uint16_t* bt, int rb, int qrow0, const uint32_t(&rnd4)[4],
                     const f32x16& s, const f32x16& dp, u32x4(&pw)[2], u32x4(&dw)[2]) __attribute__((always_inline)) {
    const int lo_r = qlo_k - (qrow0 + hf * 4), hi_r = qhi_k - (qrow0 + hf * 4);
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const f32x4 l4 = rterm(buf, 0, rb + ig * 8);
      f32x4 d4 = {};
      if constexpr (!FOLD) d4 = rterm(buf, 1, rb + ig * 8);
      u32x2 bw = {0u, 0u};
      if constexpr (BIAS) bw = bias_chunk(bt, rb, ig);
      const uint32_t rnd = rnd4[ig];  // dropout bytes of rows qrow0 + ig*8 + hf*4 + 0..3, key kj
      u32x2 pp, dd;
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2) {
        float p2[2], s2[2];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const int e = u2 * 2 + v, i = ig * 4 + e;
          const int off = ig * 8 + e;
          float pv = fast_exp2(fmaf(biased(s[i], bw, e), c, -l4[e]));
          pv = (off >= lo_r && off <= hi_r) ? pv : 0.0f;
          float pk = pv, dpz = dp[i];
          if constexpr (DROP) {
            const bool kp = drop_keep(rnd, e, dg.t);
            pk = kp ? pv : 0.0f;
            dpz = kp ? dpz * dg.scale : 0.0f;
          }
          p2[v] = pk;
          s2[v] = FOLD ? pv * dpz : pv * (dpz - d4[e]);
        }
        pp[u2] = pack_bf16(p2[0], p2[1]);
        dd[u2] = pack_bf16(s2[0], s2[1]);
      }
      // accumulator elements ig*4 .. ig*4+3 are B-operand elements
      // (ig%2)*4 .. +3 of K-step ig/2
      const int kstep = ig >> 1, e0 = (ig & 1) * 2;
      pw[kstep][e0] = pp[0];
      pw[kstep][e0 + 1] = pp[1];
      dw[kstep][e0] = dd[0];
      dw[kstep][e0 + 1] = dd[1];
    }
  };
  // C(u): dV^T (dims x keys) += dO^T P ; dK^T (dims x keys) += Q^T dS.
  auto phase_c = [&](const uint16_t* Qs, const uint16_t* Os, int rb, const u32x4(&pw)[2], const u32x4(&dw)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int pos0 = rb + kk * 16;
#pragma unroll
      for (int db = 0; db < DV / 32; ++db) dv[db] = mfma32(otr.read(Os, pos0, db), as_bf16x8(pw[kk]), dv[db]);
#pragma unroll
      for (int db = 0; db < DQK / 32; ++db) dk[db] = mfma32(qtr.read(Qs, pos0, db), as_bf16x8(dw[kk]), dk[db]);
    }
  };

  StageWalk b_walk{0, 0, T > 0 ? q_first : a.S};  // stage of the block in B
  StageWalk copy_walk = b_walk;                    // next stage to copy

  // DSOUT: each block's bf16 dS (the B operand of its dK products, which is
  // -dS under the fold, dS with dropout: ds_stored_sign) goes to block (q - q_first) / 32 of the slab
  // of (batch, head, key tile) (ds_slab; a head's slab is ds_head_blocks
  // blocks after the previous head's): wave w's 32 keys at w * 2 KiB, lane
  // l's 16 values (rows q + acc_row(i, l / 32), key l % 32, i = 0..15) at
  // l * 32 bytes.  A block is stored when some row of it sees a key of this
  // wave, i.e. when it meets the rows [ds_lo, ds_hi] that see any of the
  // wave's keys (one interval: both ends grow with the key, and a valid key
  // is seen at least by its own row) -- the test tile_class makes, with
  // which the dQ kernel decides what it reads; padding blocks (index NB and
  // up) store nothing (empty resource).  A block's dS is complete once its
  // masked redo has run, so iteration u stores block u - 1, whose registers
  // its C products read anyway (storing two blocks after each stage barrier,
  // to give the stores longer before the next copy wait, kept one block's dS
  // live an iteration longer: 8 % slower at head dim 192, no faster below).
  // Non-temporal stores (cache policy nt): the blocks are read
  // once, by the next kernel, and would otherwise push this kernel's Q / dO
  // tiles out of L2 (measured: 4-5 % on the kernel).
  constexpr int kNonTemporal = 2;
  const uint16_t* ds_base = nullptr;
  size_t ds_hstride = 0;
  int ds_lo = 1, ds_hi = 0;
  if constexpr (DSOUT) {
    int first, count;
    ds_slab(a, kt, first, count);
    ds_hstride = (size_t)a.ds_head_blocks * 4096;
    ds_base = a.ds + (size_t)(b * a.Hq + g * a.G + hs * Gs) * ds_hstride + (size_t)first * 4096;
    const int kw0 = j0 + w * 32, kw1 = (kw0 + 31 < m.L ? kw0 + 31 : m.L - 1);
    if (kw0 < m.L) {
      int lo0, hi0, lo1, hi1;
      col_query_bounds(m, kw0, lo0, hi0);
      col_query_bounds(m, kw1, lo1, hi1);
      ds_lo = lo0;
      ds_hi = hi1;
    }
  }
  // First block of the stage of the block in B (its first row is
  // b_walk.q0), and of the stage before it.
  const uint16_t* ds_cur = ds_base;
  const uint16_t* ds_prev = ds_base;
  int ds_cur_q = b_walk.q0, ds_prev_q = b_walk.q0;
  auto store_ds = [&](int blk, const uint16_t* blk_ptr, int q, const u32x4(&dw)[2]) __attribute__((always_inline)) {
    if constexpr (DSOUT) {
      const bool ok = blk >= 0 && blk < NB && q <= ds_hi && q + 31 >= ds_lo;
      const __amdgpu_buffer_rsrc_t res = buf_rsrc(blk_ptr, ok ? 8192u : 0u);
      const uint32_t off = (uint32_t)(w * 2048 + lane * 32);
      __builtin_amdgcn_raw_buffer_store_b128(dw[0], res, off, 0, kNonTemporal);
      __builtin_amdgcn_raw_buffer_store_b128(dw[1], res, off + 16, 0, kNonTemporal);
    }
  };

  // Iteration u, with P = u % 6 fixing the register sets and ring slots:
  // block u sits in slot (u/2) % 3 = (P/2) % 3 at row offset (P%2)*32.
  // The three phases are cut into four chunks, each holding a quarter of
  // A(u+1)'s and of C(u-1)'s MFMAs and one 4-row group of B(u).  Chunk k's
  // MFMA operands (and its rows' lse2 / delta) are read from LDS during
  // chunk k-1, and a scheduling fence closes each chunk, so reads stay a
  // chunk ahead of their use and register pressure stays bounded.
  constexpr int NSK = DQK / 16, NPK = DV / 16, NA = NSK + NPK;  // A: S then dP k-steps
  constexpr int NDV = DV / 32, NDK = DQK / 32, NC = 2 * (NDV + NDK);  // C: per K-step, dV then dK blocks
  constexpr int NCH = 4, EA = NA / NCH, EC = NC / NCH;
  static_assert(NA % NCH == 0 && NC % NCH == 0, "chunking");
  // Operand sets of two chunks; set 0 also carries the first chunk of the
  // next iteration, read during the last chunk of the current one.
  bf16x8 opa[2][EA], opc[2][EC];
  f32x4 l4[2], d4[2];
  f32x16 dini;  // FOLD: start of the dP accumulator of block u+1
  constexpr int KDP = NSK / EA;  // chunk whose A products start dP
  static_assert(KDP > 0, "the dP start is read a chunk ahead");
  u32x2 b4[2] = {{0u, 0u}, {0u, 0u}};  // bias of the chunk's four rows (BIAS)
  // Chunk k's LDS reads for the iteration of phase P into set st: A(u+1)'s
  // operands (RA), C(u-1)'s (RC), B(u)'s lse2 / delta (RL).
  auto read_chunk = [&](auto phase, auto kc, auto setc, auto ra, auto rc, auto rl) __attribute__((always_inline)) {
    constexpr int P = decltype(phase)::value, k = decltype(kc)::value, st = decltype(setc)::value;
    constexpr int cur = P & 1, nxt = cur ^ 1;
    constexpr int slot_u = (P >> 1) % 3, slot_n = ((P + 1) >> 1) % 3, slot_p = ((P + 5) >> 1) % 3;
    if constexpr (decltype(ra)::value) {
#pragma unroll
      for (int e = 0; e < EA; ++e) {
        const int i = k * EA + e;
        opa[st][e] = as_bf16x8(i < NSK ? rows_at(IC<slot_n * C::STAGE>{}, qrd, qrd_f, nxt * 32, i)
                                       : rows_at(IC<slot_n * C::STAGE + C::QT>{}, ord, ord_f, nxt * 32, i - NSK));
      }
      if constexpr (FOLD && k == KDP) dini = delta_init(slot_n, nxt * 32);
    }
    if constexpr (decltype(rc)::value) {
#pragma unroll
      for (int e = 0; e < EC; ++e) {
        const int i = k * EC + e, kk = i / (NDV + NDK), j = i % (NDV + NDK);
        opc[st][e] = j < NDV ? tr_at(IC<slot_p * C::STAGE + C::QT>{}, otr, otr_f, nxt * 32 + kk * 16, j)
                             : tr_at(IC<slot_p * C::STAGE>{}, qtr, qtr_f, nxt * 32 + kk * 16, j - NDV);
      }
    }
    if constexpr (decltype(rl)::value) {
      l4[st] = rterm(slot_u, 0, cur * 32 + k * 8);
      if constexpr (!FOLD) d4[st] = rterm(slot_u, 1, cur * 32 + k * 8);
      if constexpr (BIAS) b4[st] = bias_chunk(btile(slot_u), cur * 32, k);
    }
  };
  using T0 = std::false_type;
  using T1 = std::true_type;
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  using C3 = std::integral_constant<int, 3>;
  // First chunk of the iteration after the one of phase P, read ahead.  When
  // that iteration opens a stage (odd phase) its A operands are only there
  // after its barrier, so they are read then.
  auto read_ahead = [&](auto phase) __attribute__((always_inline)) {
    constexpr int PN = (decltype(phase)::value + 1) % 6;
    using PNC = std::integral_constant<int, PN>;
    if constexpr ((PN & 1) != 0) read_chunk(PNC{}, C0{}, C0{}, T0{}, T1{}, T1{});
    else read_chunk(PNC{}, C0{}, C0{}, T1{}, T1{}, T1{});
  };
  auto iteration = [&](int u, auto phase) __attribute__((always_inline)) {
    constexpr int P = decltype(phase)::value;
    constexpr int cur = P & 1, nxt = cur ^ 1;
    constexpr int slot_u = (P >> 1) % 3;
    if constexpr ((P & 1) != 0) {
      // Opens stage s = (u+1)/2: wait for its copy, then refill the slot of
      // stage s-2 (last read by C(u-2) in the previous iteration) with s+1.
      lds_dma_wait();
      __syncthreads();
      if (copy_walk.t < TP) {
        issue_stage(copy_walk, (((P + 1) >> 1) + 1) % 3);
        walk_next(copy_walk);
      }
    } else {
      walk_next(b_walk);  // block u opens a new stage
      if constexpr (DSOUT) {
        ds_prev = ds_cur;
        ds_prev_q = ds_cur_q;
        ds_cur = ds_base + (size_t)b_walk.hh * ds_hstride + (size_t)((b_walk.q0 - q_first) >> 5) * 4096;
        ds_cur_q = b_walk.q0;
      }
    }
    const int q_u = b_walk.q0 + cur * 32;  // first row of block u
    const int bh_u = b * a.Hq + g * a.G + hs * Gs + b_walk.hh;  // its (batch, query head)
    if constexpr (DSOUT) {
      // Block u-1 (set nxt, read by C(u-1) in this iteration anyway): the
      // first half of this stage (odd u) or the second half of the previous
      // one (even u).
      if constexpr ((P & 1) != 0) store_ds(u - 1, ds_cur, ds_cur_q, DW[nxt]);
      else store_ds(u - 1, ds_prev + 4096, ds_prev_q + 32, DW[nxt]);
    }
    uint32_t rnd_u[4] = {0u, 0u, 0u, 0u};
    if constexpr (DROP) drop_rows(bh_u, q_u, rnd_u);

    auto compute_chunk = [&](auto kc, auto setc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value, st = decltype(setc)::value;
#pragma unroll
      for (int e = 0; e < EC; ++e) {
        const int i = k * EC + e, kk = i / (NDV + NDK), j = i % (NDV + NDK);
        if (j < NDV) dv[j] = mfma32(opc[st][e], as_bf16x8(PW[nxt][kk]), dv[j]);
        else dk[j - NDV] = mfma32(opc[st][e], as_bf16x8(DW[nxt][kk]), dk[j - NDV]);
      }
#pragma unroll
      for (int e = 0; e < EA; ++e) {
        const int i = k * EA + e;
        if (i < NSK) S[nxt] = mfma32(opa[st][e], kreg[i], i == 0 ? f32x16{} : S[nxt]);
        else DP[nxt] = mfma32(opa[st][e], vreg[i - NSK], i == NSK ? (FOLD ? dini : f32x16{}) : DP[nxt]);
      }
      // B(u) without the mask, rows k*8 + hf*4 + 0..3 of the block:
      // accumulator elements 4k .. 4k+3, which are B-operand elements
      // (k%2)*4 .. +3 of K-step k/2.  Blocks that need the mask redo B below.
      u32x2 pp, dd;
      const uint32_t rnd = rnd_u[k];  // dropout bytes of rows q_u + k*8 + hf*4 + 0..3, key kj
#pragma unroll
      for (int u2 = 0; u2 < 2; ++u2) {
        float p2[2], s2[2];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const int e = u2 * 2 + v, i = k * 4 + e;
          const float pv = fast_exp2(fmaf(biased(S[cur][i], b4[st], e), c, -l4[st][e]));
          float pk = pv, dpz = DP[cur][i];
          if constexpr (DROP) {
            const bool kp = drop_keep(rnd, e, dg.t);
            pk = kp ? pv : 0.0f;
            dpz = kp ? dpz * dg.scale : 0.0f;
          }
          p2[v] = pk;
          s2[v] = FOLD ? pv * dpz : pv * (dpz - d4[st][e]);
        }
        pp[u2] = pack_bf16(p2[0], p2[1]);
        dd[u2] = pack_bf16(s2[0], s2[1]);
      }
      // Pin the results here: without it the compiler sinks this softmax
      // work next to its consumer, C in the next iteration, which serialises
      // it with those MFMAs again.
      asm volatile("" : "+v"(pp), "+v"(dd));
      constexpr int kstep = k >> 1, e0 = (k & 1) * 2;
      PW[cur][kstep][e0] = pp[0];
      PW[cur][kstep][e0 + 1] = pp[1];
      DW[cur][kstep][e0] = dd[0];
      DW[cur][kstep][e0 + 1] = dd[1];
    };
    // Within a chunk: each MFMA followed by LDS reads and VALU work, so the
    // next MFMA is not issued while the matrix unit is still busy (a stalled
    // MFMA would hold up every instruction behind it).
    auto pattern = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < EA + EC; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);               // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, SDPA_DKDV_DS, 0);    // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, SDPA_DKDV_VALU, 0);  // VALU
      }
    };
    using PC = std::integral_constant<int, P>;
    // Chunk 0's operands were read during the previous iteration, except A's
    // after a barrier: C's MFMAs come first in each chunk and cover them.
    if constexpr ((P & 1) != 0) read_chunk(PC{}, C0{}, C0{}, T1{}, T0{}, T0{});
    read_chunk(PC{}, C1{}, C1{}, T1{}, T1{}, T1{});
    compute_chunk(C0{}, C0{});
    pattern();
    __builtin_amdgcn_sched_barrier(0);
    read_chunk(PC{}, C2{}, C0{}, T1{}, T1{}, T1{});
    compute_chunk(C1{}, C1{});
    pattern();
    __builtin_amdgcn_sched_barrier(0);
    read_chunk(PC{}, C3{}, C1{}, T1{}, T1{}, T1{});
    compute_chunk(C2{}, C0{});
    pattern();
    __builtin_amdgcn_sched_barrier(0);
    read_ahead(PC{});
    compute_chunk(C3{}, C1{});
    pattern();
    __builtin_amdgcn_sched_barrier(0);
    // Blocks that some of this wave's (row, key) pairs cannot see (diagonal,
    // window edge, padding): redo B with the mask.
    if (!(q_u >= all_lo && q_u + 31 <= all_hi))
      phase_b(slot_u, btile(slot_u), cur * 32, q_u, rnd_u, S[cur], DP[cur], PW[cur], DW[cur]);
  };

  if (NB > 0) {
    issue_stage(b_walk, 0);
    StageWalk copy_walk_1 = b_walk;
    walk_next(copy_walk_1);
    issue_stage(copy_walk_1, 1);
    copy_walk = copy_walk_1;
    walk_next(copy_walk);
    lds_dma_wait();
    __syncthreads();
    // Block 0 has no predecessor: A(0), then A(1) with B(0).
    phase_a(qtile(0), otile(0), 0, S[0], DP[0]);
    phase_a(qtile(0), otile(0), 32, S[1], DP[1]);
    uint32_t rnd_0[4] = {0u, 0u, 0u, 0u};
    if constexpr (DROP) drop_rows(b * a.Hq + g * a.G + hs * Gs + b_walk.hh, b_walk.q0, rnd_0);
    phase_b(0, btile(0), 0, b_walk.q0, rnd_0, S[0], DP[0], PW[0], DW[0]);
    read_ahead(std::integral_constant<int, 0>{});  // first chunk of iteration 1
    // Iterations 1 .. NI in trips of six (one per phase), padded past the
    // last block NB-1 with empty blocks: their stages copy rows past the
    // valid length, so Q, dO, lse2 and delta arrive as zeros, the mask
    // zeroes P, and C adds exact zeros.  A single code path per trip keeps
    // every register set in place.
    for (int u = 1; u <= NI; u += 6) {
      iteration(u, std::integral_constant<int, 1>{});
      iteration(u + 1, std::integral_constant<int, 2>{});
      iteration(u + 2, std::integral_constant<int, 3>{});
      iteration(u + 3, std::integral_constant<int, 4>{});
      iteration(u + 4, std::integral_constant<int, 5>{});
      iteration(u + 5, std::integral_constant<int, 0>{});
    }
    // Block NI (even, first half of stage NI/2, ring slot 0) still owes C.
    phase_c(qtile(0), otile(0), 0, PW[0], DW[0]);
    store_ds(NI, ds_cur, ds_cur_q, DW[0]);  // block NI (set 0)
  }

  // Epilogue: lane owns key kj, dims db*32 + acc_row(i, hf).
  // dK / dV rows exist up to the batch's row count (S, or the segment size
  // of packed tensors); the fp32 partials always use the padded layout.
  if (kj < seq_rows(a, b)) {
    if (nsp == 1) {
      uint16_t* dkp = static_cast<uint16_t*>(a.dk) + ((seq_row0(a, b) + kj) * a.Hkv + g) * DQK + hf * 4;
      uint16_t* dvp = static_cast<uint16_t*>(a.dv) + ((seq_row0(a, b) + kj) * a.Hkv + g) * DV + hf * 4;
#pragma unroll
      for (int db = 0; db < DQK / 32; ++db)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const float ks = FOLD ? -a.scale : a.scale;
          u32x2 val = {pack_bf16(dk[db][ig * 4] * ks, dk[db][ig * 4 + 1] * ks),
                       pack_bf16(dk[db][ig * 4 + 2] * ks, dk[db][ig * 4 + 3] * ks)};
          *reinterpret_cast<u32x2*>(dkp + db * 32 + ig * 8) = val;
        }
#pragma unroll
      for (int db = 0; db < DV / 32; ++db)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const float zs = DROP ? dg.scale : 1.0f;
          u32x2 val = {pack_bf16(dv[db][ig * 4] * zs, dv[db][ig * 4 + 1] * zs),
                       pack_bf16(dv[db][ig * 4 + 2] * zs, dv[db][ig * 4 + 3] * zs)};
          *reinterpret_cast<u32x2*>(dvp + db * 32 + ig * 8) = val;
        }
    } else {
      // fp32 partials of this split (dK without the softmax scale, dV without
      // the dropout scale), same element order as dK / dV.
      const size_t row = ((size_t)(hs * a.B + b) * a.S + kj) * a.Hkv + g;
      float* dkp = a.kv_part + row * DQK + hf * 4;
      float* dvp = a.kv_part + (size_t)nsp * a.B * a.S * a.Hkv * DQK + row * DV + hf * 4;
#pragma unroll
      for (int db = 0; db < DQK / 32; ++db)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig)
          *reinterpret_cast<f32x4*>(dkp + db * 32 + ig * 8) =
              FOLD ? -f32x4{dk[db][ig * 4], dk[db][ig * 4 + 1], dk[db][ig * 4 + 2], dk[db][ig * 4 + 3]}
                   : f32x4{dk[db][ig * 4], dk[db][ig * 4 + 1], dk[db][ig * 4 + 2], dk[db][ig * 4 + 3]};
#pragma unroll
      for (int db = 0; db < DV / 32; ++db)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig)
          *reinterpret_cast<f32x4*>(dvp + db * 32 + ig * 8) =
              f32x4{dv[db][ig * 4], dv[db][ig * 4 + 1], dv[db][ig * 4 + 2], dv[db][ig * 4 + 3]};
    }
  }
}

// dst[i] = bf16(mul * sum over splits s = 0 .. n_splits-1 of part[s*n + i]),
// four consecutive elements per thread (n and row_elems are multiples of 4).
// The partials use the padded layout, row b*S + j of row_elems elements; for
// packed (THD) tensors that row goes to row seq_offsets[b] + j of dst, and
// rows past the segment size are not written.
__global__ __launch_bounds__(256) void dkdv_split_reduce_kernel(const float* part, uint16_t* dst, size_t n, int n_splits,
                                                                float mul, const int32_t* seq_offsets, int S,
                                                                int row_elems) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
  size_t out = i;
  if (seq_offsets) {
    const size_t r = i / (size_t)row_elems;
    const int b = (int)(r / (size_t)S), j = (int)(r % (size_t)S);
    const int rows = seq_offsets[b + 1] - seq_offsets[b];
    if (j >= rows) return;
    out = ((size_t)seq_offsets[b] + j) * row_elems + (i - r * row_elems);
  }
  f32x4 acc = *reinterpret_cast<const f32x4*>(part + i);
  for (int sp = 1; sp < n_splits; ++sp) acc += *reinterpret_cast<const f32x4*>(part + (size_t)sp * n + i);
  *reinterpret_cast<u32x2*>(dst + out) = u32x2{pack_bf16(acc[0] * mul, acc[1] * mul), pack_bf16(acc[2] * mul, acc[3] * mul)};
}

// Explicit instantiations: with only the implicit ones from the launchers
// below, the host pass of this compiler drops the launch stub of the last
// kernel instantiated in the file.
template __global__ void bwd_dkdv_bf16_kernel<64, 64, false, false, false>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<128, 128, false, false, false>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<192, 128, false, false, false>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<64, 64, true, false, false>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<128, 128, true, false, false>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<192, 128, true, false, false>(KArgs);
// Stored-dS variants (with dropout and / or a bias; a bias at head dims 64 and 128).
template __global__ void bwd_dkdv_bf16_kernel<64, 64, false, false, true>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<128, 128, false, false, true>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<192, 128, false, false, true>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<64, 64, false, true, true>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<128, 128, false, true, true>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<64, 64, true, false, true>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<128, 128, true, false, true>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<192, 128, true, false, true>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<64, 64, true, true, true>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<128, 128, true, true, true>(KArgs);
// Bias variants: a stage grows by a 64 x 128 bf16 tile (147 KB of LDS in all
// at head dim 128; the 192-dim stages would not fit).
template __global__ void bwd_dkdv_bf16_kernel<64, 64, false, true, false>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<128, 128, false, true, false>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<64, 64, true, true, false>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<128, 128, true, true, false>(KArgs);

// The variant for a's dropout and bias; DSOUT: the stored-dS one.
template <int DQK, int DV, bool DSOUT>
static hipError_t launch_dkdv_variant(const KArgs& a, dim3 grid, hipStream_t stream) {
  constexpr int NT = DkdvCfg<DQK, DV, false>::NT;
  if constexpr (DQK <= 128) {
    static_assert(DkdvCfg<DQK, DV, true>::LDS_ELEMS * 2 <= 160 * 1024, "bias stages fit the LDS");
    if (a.bias) {
      if (a.drop_t > 0) hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<DQK, DV, true, true, DSOUT>), grid, dim3(NT), 0, stream, a);
      else hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<DQK, DV, false, true, DSOUT>), grid, dim3(NT), 0, stream, a);
      return hipGetLastError();
    }
  } else if (a.bias) {
    return hipErrorInvalidValue;  // no bias variant for these head dims
  }
  if (a.drop_t > 0) hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<DQK, DV, true, false, DSOUT>), grid, dim3(NT), 0, stream, a);
  else hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<DQK, DV, false, false, DSOUT>), grid, dim3(NT), 0, stream, a);
  return hipGetLastError();
}

template <int DQK, int DV>
static hipError_t launch_dkdv_cfg(KArgs a, hipStream_t stream) {
  using D = DkdvCfg<DQK, DV, false>;
  static_assert(D::BN == kDkdvKeyTile, "split rule uses the kernel's key tile");
  const int nkt = (a.S + D::BN - 1) / D::BN;
  const dim3 grid((unsigned)(nkt * a.B * a.Hkv * a.n_splits));
  return a.ds ? launch_dkdv_variant<DQK, DV, true>(a, grid, stream) : launch_dkdv_variant<DQK, DV, false>(a, grid, stream);
}

int dkdv_head_splits(int B, int S, int Hkv, int G, bool causal, int wl, int wr, int dqk, int dv) {
  const long long base = (long long)((S + kDkdvKeyTile - 1) / kDkdvKeyTile) * B * Hkv;
  // Most 32-row blocks one workgroup walks per query head: rows j0-wr ..
  // j0+127+wl of a key tile (causal: from j0), in 64-row stages.
  const long long before = causal ? 0 : (wr < 0 ? S : wr), after = wl < 0 ? S : wl;
  long long span = before + kDkdvKeyTile + after;
  if (span > S) span = S;
  long long stages = (span + 63) / 64 + 1;
  if (stages > (S + 63) / 64) stages = (S + 63) / 64;
  auto fits = [&](int d) __attribute__((always_inline)) { return base * d >= kDkdvMinGrid && 2 * stages * (G / d) <= kDkdvMaxBlocks; };
  int want = G;
  for (int d = 1; d <= G; ++d)
    if (G % d == 0 && fits(d)) {
      want = d;
      break;
    }
  // The fp32 partials must stay within kDkdvMaxPartialBytes: else the
  // largest divisor below the wanted count that does.
  const long long per_split = (long long)B * S * Hkv * (dqk + dv) * 4;
  for (int d = want; d > 1; --d)
    if (G % d == 0 && per_split * d <= kDkdvMaxPartialBytes) return d;
  return 1;
}

hipError_t launch_dkdv_split_reduce(const KArgs& a, int dqk, int dv, hipStream_t stream) {
  const size_t rows = (size_t)a.B * a.S * a.Hkv;
  const size_t nk = rows * dqk, nv = rows * dv;
  hipLaunchKernelGGL(dkdv_split_reduce_kernel, dim3((unsigned)((nk / 4 + 255) / 256)), dim3(256), 0, stream,
                     a.kv_part, static_cast<uint16_t*>(a.dk), nk, a.n_splits, a.scale, a.seq_offsets, a.S,
                     a.Hkv * dqk);
  hipLaunchKernelGGL(dkdv_split_reduce_kernel, dim3((unsigned)((nv / 4 + 255) / 256)), dim3(256), 0, stream,
                     a.kv_part + (size_t)a.n_splits * nk, static_cast<uint16_t*>(a.dv), nv, a.n_splits,
                     a.drop_t > 0 ? a.drop_scale : 1.0f,
                     a.seq_offsets, a.S, a.Hkv * dv);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const KArgs& a, int dqk, int dv, hipStream_t stream) {
  if (dqk == 64 && dv == 64) return launch_dkdv_cfg<64, 64>(a, stream);
  if (dqk == 128 && dv == 128) return launch_dkdv_cfg<128, 128>(a, stream);
  if (dqk == 192 && dv == 128) return launch_dkdv_cfg<192, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace sdpa
