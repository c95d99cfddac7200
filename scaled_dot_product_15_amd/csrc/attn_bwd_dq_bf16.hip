// Backward attention, dQ, bf16 inputs, fp32 accumulation, gfx950 MFMA 32x32x16,
// with the backward pre-pass (delta, lse2, sink-gradient partials) fused in.
//
// With P = exp(scale * Q K^T - LSE) recomputed from the forward's LSE and
// delta_i = rowsum(dO * O) from the pre-pass (PR #2225 backward: dz = dO in,
// grad_q, grad_k, grad_v out):
//     dP = dO V^T,  dS = P * (dP - delta),
//     dV = P^T dO,  dK = scale * dS^T Q,  dQ = scale * dS K.
// This kernel (deterministic, no atomics): a workgroup owns BM = 128 query
// rows of one (batch, query head) and walks the visible key tiles, keeping dQ
// in registers; it recomputes S and dP instead of sharing them with the dK/dV
// kernel, which would need atomics on dQ.
// MFMA operand layouts: a lane of a 32x32 accumulator owns one column and 16
// rows (acc_row).  Contractions over head dims read 16-byte row pieces of a
// swizzled row-major LDS tile; contractions over the sequence take the
// accumulator-side operand straight from registers and the other one with
// LDS transpose loads from the same tile (TrReads).  Tiles arrive by
// direct memory-to-LDS copies, double buffered, one barrier per step.
//
// DROP (attention dropout, dropout.h): with Z = keep / (1 - p),
// dS = P * (Z dP - delta); delta = rowsum(dO * O) already holds the dropped O.
//
// BIAS (additive post-scale attention bias): P = exp(scale q.k + bias - LSE);
// bias / scale is added to the recomputed scores; each lane loads its row's
// bias values of a key tile at the start of that tile's step (RowBias).  For
// a bias that is not shared (one matrix per batch and head) dBias = dS: the
// kernel writes each tile's bf16 dS (the values the dQ products take) to its
// rows of dBias, and zeros for the keys its rows do not reach.
#include <type_traits>

#include "dropout.h"
#include "launch.h"

// Tile parameters (build-time overridable for tuning sweeps).
#ifndef SDPA_DQ_BN
#define SDPA_DQ_BN 64
#endif
#ifndef SDPA_DQ_WAVES
#define SDPA_DQ_WAVES 4
#endif

namespace sdpa {

// -------------------------------------------------------------------- dQ ---

template <int DQK, int DV>
struct DqCfg {
  static constexpr int BM = 32 * SDPA_DQ_WAVES;  // query rows per workgroup (32 per wave)
  static constexpr int BN = SDPA_DQ_BN;  // keys per step
  static constexpr int NT = 64 * SDPA_DQ_WAVES;
  static constexpr int KCH = DQK / 8, VCH = DV / 8;
  static constexpr int KT = BN * DQK, VT = BN * DV;
  static constexpr int LDS_ELEMS = 2 * (KT + VT);
};

// The dropout and the bias variants are held to two workgroups per CU (head
// dims up to 128) so two waves share each SIMD as in the plain kernel; with
// both, the register budget of two does not hold and the bound is one.
template <int DQK, int DV, bool DROP, bool BIAS>
__global__ __launch_bounds__(64 * SDPA_DQ_WAVES, ((DROP != BIAS) && DQK <= 128) ? 2 : 1) void bwd_dq_bf16_kernel(KArgs a) {
  using C = DqCfg<DQK, DV>;
  // Without dropout or bias (and below 192 dims, whose registers are
  // full), delta is folded into the dP products: the accumulator starts at
  // delta (a loop-invariant register block) and dO enters negated, so it
  // ends at delta - dP and P times it is -dS with no subtraction; dQ then
  // accumulates -dQ, negated by the final scale (exact sign changes).
  constexpr bool FOLD = !DROP && !BIAS && DQK <= 128;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  auto ktile = [&](int buf) __attribute__((always_inline)) { return lds + buf * (C::KT + C::VT); };
  auto vtile = [&](int buf) __attribute__((always_inline)) { return lds + buf * (C::KT + C::VT) + C::KT; };

  const int tid = threadIdx.x, w = wave_id(tid), lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  // Same tile order as the forward (q_tile_of).  Below 128 dims it is
  // written here through xcd_group_item (groups of the G heads of one query
  // tile; the same assignment q_tile_of computes): with that arithmetic the
  // compiler fits the 64-dim kernel in 168 registers, three waves per SIMD
  // instead of two (dQ 5-7 % faster on the 64-dim sweep).
  int b, h, qt;
  if constexpr (kGroupedOrder<DQK>) {
    q_tile_of<true>(a, blockIdx.x, b, h, qt);
  } else {
    int grp, item;
    xcd_group_item(blockIdx.x, a.B * a.Hkv * a.n_tiles, a.G, grp, item);
    const int per_tile = a.B * a.Hkv;
    qt = a.n_tiles - 1 - grp / per_tile;
    b = (grp % per_tile) / a.Hkv;
    h = (grp % per_tile) % a.Hkv * a.G + item;
  }
  const int g = h / a.G;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  const int bh = b * a.Hq + h;
  const DropGen dg = drop_gen(a);
  const int i0 = qt * C::BM, qw0 = i0 + w * 32, qi = qw0 + l32;
  int klo, khi;
  row_key_bounds(m, qi, klo, khi);

  bf16x8 qreg[DQK / 16], oreg[DV / 16];
  float lse2 = 0.0f, dl = 0.0f;
  {
    const size_t qstride = (size_t)a.Hq * DQK, ostride = (size_t)a.Hq * DV;
    const __amdgpu_buffer_rsrc_t qres = buf_rsrc(static_cast<const uint16_t*>(a.q) + (seq_row0(a, b) * a.Hq + h) * DQK,
                                                 (uint32_t)(m.L * qstride * 2));
    const __amdgpu_buffer_rsrc_t ores = buf_rsrc(static_cast<const uint16_t*>(a.d_o) + (seq_row0(a, b) * a.Hq + h) * DV,
                                                 (uint32_t)(m.L * ostride * 2));
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks)
      qreg[ks] = as_bf16x8(buf_load16(qres, (uint32_t)(qi * qstride + ks * 16 + hf * 8) * 2));
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
      oreg[ks] = as_bf16x8(buf_load16(ores, (uint32_t)(qi * ostride + ks * 16 + hf * 8) * 2));
    // Backward pre-pass for this wave's 32 rows, fused here: delta =
    // rowsum(dO * O) (each lane half holds half of the row's dims; rows
    // >= L read zeros), lse2 = LSE * log2(e) (0 past L), both stored for the
    // dK/dV kernel; for a sink logit z, the partial sum over the 32 rows of
    // dL/dz_i = -exp(z - LSE_i) delta_i (the sink enters only the softmax
    // denominator), added up over the rows' chunks in fixed order later.
    const __amdgpu_buffer_rsrc_t outres = buf_rsrc(static_cast<const uint16_t*>(a.o) + (seq_row0(a, b) * a.Hq + h) * DV,
                                                   (uint32_t)(m.L * ostride * 2));
    float part = 0.0f;
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks) {
      const u32x4 ov = buf_load16(outres, (uint32_t)(qi * ostride + ks * 16 + hf * 8) * 2);
      const u32x4 dv4 = __builtin_bit_cast(u32x4, oreg[ks]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        part += __builtin_bit_cast(float, ov[e] << 16) * __builtin_bit_cast(float, dv4[e] << 16);
        part += __builtin_bit_cast(float, ov[e] & 0xffff0000u) * __builtin_bit_cast(float, dv4[e] & 0xffff0000u);
      }
    }
    dl = halves_sum(part);
    const size_t row = ((size_t)b * a.Hq + h) * a.S + qi;
    const float lse_nat = qi < m.L ? a.lse[row] : 0.0f;
    lse2 = qi < m.L ? lse_nat * kLog2e : 0.0f;
    if (hf == 0 && qi < a.S) {
      a.delta[row] = dl;
      a.lse2[row] = lse2;
    }
    if (a.softmax_type != 0) {
      float dz = (hf == 0 && qi < m.L) ? -expf(sink_logit(a, h) - lse_nat) * dl : 0.0f;
#pragma unroll
      for (int off = 16; off > 0; off >>= 1) dz += __shfl_xor(dz, off);
      if (lane == 0 && qw0 < a.S) a.dz_partial[((size_t)b * a.Hq + h) * a.n_chunks + qw0 / 32] = dz;
    }
  }
  f32x16 dq[DQK / 32];
#pragma unroll
  for (int i = 0; i < DQK / 32; ++i) dq[i] = f32x16{};
  // -dO^T for the folded dP products.
  bf16x8 oneg[DV / 16];
#pragma unroll
  for (int ks = 0; ks < DV / 16; ++ks) oneg[ks] = as_bf16x8(__builtin_bit_cast(u32x4, oreg[ks]) ^ 0x80008000u);

  int lo = 0, hi = -1;
  const int nrow = (i0 + C::BM < m.L ? i0 + C::BM : m.L) - 1;
  if (!key_range(m, i0, nrow, lo, hi)) { lo = 0; hi = -1; }
  const int kt0 = lo / C::BN, kt1 = hi < 0 ? -1 : hi / C::BN;
  RowBias<C::BN / 32> bias;
  if constexpr (BIAS) bias.init(a, b, h, qi, hf);

  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + (seq_row0(a, b) * a.Hkv + g) * DQK;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v) + (seq_row0(a, b) * a.Hkv + g) * DV;
  const size_t kstride = (size_t)a.Hkv * DQK, vstride = (size_t)a.Hkv * DV;
  const TileCopy<C::BN, C::KCH, C::NT> kcopy(tid, (uint32_t)(kstride * 2));
  const TileCopy<C::BN, C::VCH, C::NT> vcopy(tid, (uint32_t)(vstride * 2));
  const RowReads<C::KCH> krd(lane);
  const RowReads<C::VCH> vrd(lane);
  const TrReads<C::KCH> ktr(lane);
  auto issue_tile = [&](int j0, int buf) __attribute__((always_inline)) {
    kcopy.issue(Kg, (uint32_t)(kstride * 2), j0, m.L, ktile(buf));
    vcopy.issue(Vg, (uint32_t)(vstride * 2), j0, m.L, vtile(buf));
  };

  // Unshared bias (dBias written here): this lane's row of dBias, and zeros
  // for keys [k0, k1) of the wave's 32 rows (16-byte stores, lanes across
  // keys; S is a multiple of 8, so every 8-key piece below S is whole).
  // (a null base and size when there is no such bias: nothing is stored then)
  const __amdgpu_buffer_rsrc_t dbias_res =
      buf_rsrc(BIAS && a.dbias_direct ? static_cast<uint16_t*>(a.d_bias) + (size_t)bh * a.S * a.S : nullptr,
               BIAS && a.dbias_direct ? (uint32_t)((size_t)a.S * a.S * 2) : 0u);
  // byte offset of (row qi, key hf*4) in this (b, h)'s matrix; rows past S store nothing
  const uint32_t dbias_off = qi < a.S ? (uint32_t)((qi * a.S + hf * 4) * 2) : 0u;
  auto dbias_zero = [&](int k0, int k1) __attribute__((always_inline)) {
    if (!a.dbias_direct) return;
    k1 = k1 < a.S ? k1 : a.S;
    uint16_t* base = static_cast<uint16_t*>(a.d_bias) + (size_t)bh * a.S * a.S;
    for (int r = 0; r < 32; ++r) {
      const int row = qw0 + r;
      if (row >= a.S) break;
      for (int k = k0 + lane * 8; k < k1; k += 64 * 8)
        *reinterpret_cast<u32x4*>(base + (size_t)row * a.S + k) = u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto tile = [&](int j0, const uint16_t* Ks, const uint16_t* Vs, auto masked) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    // Element i of block kb: key j0 + hf*4 + kb*32 + acc_row(i, 0), query qi.
    const int base = j0 + hf * 4;
    // Dropout bytes of keys base + kb*32 + g*8 + 0..3, drawn before the score
    // products so the generator's temporaries are dead while S and dP live.
    uint32_t rnd[C::BN / 32][4];
    if constexpr (DROP) {
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb) drop_rows_quad(dg, bh, qi, base + kb * 32, rnd[kb]);
    }
    f32x16 st[C::BN / 32], dpt[C::BN / 32];
#pragma unroll
    for (int kb = 0; kb < C::BN / 32; ++kb) {
      st[kb] = f32x16{};
      if constexpr (FOLD) {
#pragma unroll
        for (int i = 0; i < 16; ++i) dpt[kb][i] = dl;
      } else {
        dpt[kb] = f32x16{};
      }
    }
    prio_mfma();
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb)
        st[kb] = mfma32(as_bf16x8(krd.read(Ks, kb * 32, ks)), qreg[ks], st[kb]);
    // This tile's bias (requested at the start of the step) joins the scores
    // while the dP products run.
    if constexpr (BIAS) bias.add(st, a.inv_scale);
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb)
        dpt[kb] = mfma32(as_bf16x8(vrd.read(Vs, kb * 32, ks)), FOLD ? oneg[ks] : oreg[ks], dpt[kb]);
    prio_valu();
    const int lo_r = klo - base, hi_r = khi - base;
    bf16x8 dsb[C::BN / 16];
#pragma unroll
    for (int kb = 0; kb < C::BN / 32; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int i = half * 8 + 2 * e + u;
            float pv = fast_exp2(fmaf(st[kb][i], a.scale_log2, -lse2));
            if constexpr (MASKED) {
              const int off = kb * 32 + (i >> 2) * 8 + (i & 3);
              pv = (off >= lo_r && off <= hi_r) ? pv : 0.0f;
            }
            float dpz = dpt[kb][i];
            if constexpr (DROP) dpz = drop_keep(rnd[kb][i >> 2], i & 3, dg.t) ? dpz * dg.scale : 0.0f;
            v2[u] = FOLD ? pv * dpz : pv * (dpz - dl);
          }
          t[e] = pack_bf16(v2[0], v2[1]);
        }
        dsb[kb * 2 + half] = as_bf16x8(t);
      }
    if constexpr (BIAS) {
      // Unshared bias: dBias = dS, row qi, keys j0 + kb*32 + hf*4 + 16 half
      // + {0..3} and + 8 + {0..3} (words 0-1 and 2-3 of dsb[kb*2 + half]).
      if (a.dbias_direct && qi < a.S) {
#pragma unroll
        for (int kb = 0; kb < C::BN / 32; ++kb)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const u32x4 wds = __builtin_bit_cast(u32x4, dsb[kb * 2 + half]);
            const int k0 = j0 + kb * 32 + half * 16;  // (+ hf * 4, in dbias_off)
            if (k0 < a.S)
              __builtin_amdgcn_raw_buffer_store_b64(u32x2{wds[0], wds[1]}, dbias_res, dbias_off + k0 * 2, 0, 0);
            if (k0 + 8 < a.S)
              __builtin_amdgcn_raw_buffer_store_b64(u32x2{wds[2], wds[3]}, dbias_res, dbias_off + (k0 + 8) * 2, 0, 0);
          }
      }
    }
    // dQ^T (dims x queries) += K^T dS^T
    prio_mfma();
#pragma unroll
    for (int kk = 0; kk < C::BN / 16; ++kk)
#pragma unroll
      for (int db = 0; db < DQK / 32; ++db)
        dq[db] = mfma32(ktr.read(Ks, kk * 16, db), dsb[kk], dq[db]);
    prio_valu();
  };

  // Same walk as the forward: tiles in pairs (buffers 0, 1, so every LDS
  // offset is a compile-time constant); key tiles every row of the
  // workgroup sees in full run unmasked, the rest masked with per-wave
  // skipping, each in a loop of its own so the dQ accumulators stay in
  // place.
  int fa = kt0, fb = kt0;  // unmasked tiles [fa, fb); fa - kt0, fb - fa even
  {
    int f0, f1;
    if (kt0 <= kt1 && full_key_tiles(m, i0, C::BM, C::BN, f0, f1)) {
      if (f0 < kt0) f0 = kt0;
      if (f1 > kt1) f1 = kt1;
      const int first = kt0 + ((f0 - kt0 + 1) & ~1);
      const int n = (f1 + 1 - first) & ~1;
      if (n > 0) {
        fa = first;
        fb = first + n;
      }
    }
  }
  auto step = [&](int kt, auto bufc, auto masked) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    const int j0 = kt * C::BN;
    // The bias loads go out before the next tile's copies: the compiler's
    // wait for them then counts only the copies issued after them.
    if constexpr (BIAS) bias.load(j0);
    if (kt < kt1) issue_tile(j0 + C::BN, buf ^ 1);
    if constexpr (decltype(masked)::value) {
      if (tile_class(m, qw0, 32, j0, C::BN) != TILE_SKIP) tile(j0, ktile(buf), vtile(buf), std::true_type{});
      else if constexpr (BIAS) dbias_zero(j0, j0 + C::BN);  // no row of this wave sees the tile
    } else {
      tile(j0, ktile(buf), vtile(buf), std::false_type{});
    }
    lds_dma_wait();
    __syncthreads();
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  if (kt0 <= kt1) issue_tile(kt0 * C::BN, 0);
  lds_dma_wait();
  __syncthreads();
  for (int kt = kt0; kt < fa; kt += 2) {
    step(kt, B0{}, std::true_type{});
    step(kt + 1, B1{}, std::true_type{});
  }
  for (int kt = fa; kt < fb; kt += 2) {
    step(kt, B0{}, std::false_type{});
    step(kt + 1, B1{}, std::false_type{});
  }
  for (int kt = fb; kt <= kt1; kt += 2) {
    step(kt, B0{}, std::true_type{});
    if (kt + 1 <= kt1) step(kt + 1, B1{}, std::true_type{});
  }

  if constexpr (BIAS) {
    // keys outside the visited tiles [kt0, kt1]
    if (kt0 <= kt1) {
      dbias_zero(0, kt0 * C::BN);
      dbias_zero((kt1 + 1) * C::BN, a.S);
    } else {
      dbias_zero(0, a.S);
    }
  }
  if (qi < seq_rows(a, b)) {
    uint16_t* dqp = static_cast<uint16_t*>(a.dq) + ((seq_row0(a, b) + qi) * a.Hq + h) * DQK + hf * 4;
#pragma unroll
    for (int db = 0; db < DQK / 32; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const float qs = FOLD ? -a.scale : a.scale;
        u32x2 val = {pack_bf16(dq[db][ig * 4] * qs, dq[db][ig * 4 + 1] * qs),
                     pack_bf16(dq[db][ig * 4 + 2] * qs, dq[db][ig * 4 + 3] * qs)};
        *reinterpret_cast<u32x2*>(dqp + db * 32 + ig * 8) = val;
      }
  }
}

// Explicit instantiations: with only the implicit ones from the launchers
// below, the host pass of this compiler drops the launch stub of the last
// kernel instantiated in the file.
template __global__ void bwd_dq_bf16_kernel<64, 64, false, false>(KArgs);
template __global__ void bwd_dq_bf16_kernel<128, 128, false, false>(KArgs);
template __global__ void bwd_dq_bf16_kernel<192, 128, false, false>(KArgs);
template __global__ void bwd_dq_bf16_kernel<64, 64, true, false>(KArgs);
template __global__ void bwd_dq_bf16_kernel<128, 128, true, false>(KArgs);
template __global__ void bwd_dq_bf16_kernel<192, 128, true, false>(KArgs);
template __global__ void bwd_dq_bf16_kernel<64, 64, false, true>(KArgs);
template __global__ void bwd_dq_bf16_kernel<128, 128, false, true>(KArgs);
template __global__ void bwd_dq_bf16_kernel<64, 64, true, true>(KArgs);
template __global__ void bwd_dq_bf16_kernel<128, 128, true, true>(KArgs);

template <int DQK, int DV>
static hipError_t launch_dq_cfg(KArgs a, hipStream_t stream) {
  using Q = DqCfg<DQK, DV>;
  a.n_tiles = (a.S + Q::BM - 1) / Q::BM;
  const dim3 grid((unsigned)(a.n_tiles * a.B * a.Hq));
  if constexpr (DQK <= 128) {
    if (a.bias) {
      if (a.drop_t > 0) hipLaunchKernelGGL((bwd_dq_bf16_kernel<DQK, DV, true, true>), grid, dim3(Q::NT), 0, stream, a);
      else hipLaunchKernelGGL((bwd_dq_bf16_kernel<DQK, DV, false, true>), grid, dim3(Q::NT), 0, stream, a);
      return hipGetLastError();
    }
  } else if (a.bias) {
    return hipErrorInvalidValue;  // no bias variant for these head dims
  }
  if (a.drop_t > 0) hipLaunchKernelGGL((bwd_dq_bf16_kernel<DQK, DV, true, false>), grid, dim3(Q::NT), 0, stream, a);
  else hipLaunchKernelGGL((bwd_dq_bf16_kernel<DQK, DV, false, false>), grid, dim3(Q::NT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16(const KArgs& a, int dqk, int dv, hipStream_t stream) {
  if (dqk == 64 && dv == 64) return launch_dq_cfg<64, 64>(a, stream);
  if (dqk == 128 && dv == 128) return launch_dq_cfg<128, 128>(a, stream);
  if (dqk == 192 && dv == 128) return launch_dq_cfg<192, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace sdpa
