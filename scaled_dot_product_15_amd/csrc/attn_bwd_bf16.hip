// Backward attention, bf16 inputs, fp32 accumulation, gfx950 MFMA 32x32x16.
//
// With P = exp(scale * Q K^T - LSE) recomputed from the forward's LSE and
// delta_i = rowsum(dO * O) from the pre-pass (PR #2225 backward: dz = dO in,
// grad_q, grad_k, grad_v out):
//     dP = dO V^T,  dS = P * (dP - delta),
//     dV = P^T dO,  dK = scale * dS^T Q,  dQ = scale * dS K.
// Two kernels, both deterministic (no atomics):
//   dkdv: a workgroup owns BN = 128 keys of one (batch, KV head); each wave
//         owns 32 keys and keeps dK, dV in registers while the workgroup walks
//         the G query heads of the group in ascending order and, for each, the
//         visible query tiles in ascending order; the GQA sum is therefore a
//         fixed-order register accumulation.
//   dq:   a workgroup owns BM = 128 query rows of one (batch, query head) and
//         walks the visible key tiles, keeping dQ in registers.
// MFMA operand layouts: a lane of a 32x32 accumulator owns one column and 16
// rows (acc_row).  Contractions over head dims read 16-byte row pieces from a
// row-major LDS tile whose rows sit 16 B apart mod 256 B; contractions over
// the sequence take the accumulator-side operand straight from registers and
// the other one with LDS transpose loads (lds_tr_operand) from a second
// row-major copy whose pitch puts the four rows of a transpose load 64 B
// apart mod 256 B.  Staging is plain row copies: no transposed stores.
#include <type_traits>

#include "launch.h"

namespace sdpa {

// Copies of a row-major tile: NP-pitch for row reads, TP-pitch for transpose loads.
template <int D>
struct TilePitch {
  static constexpr int NP = D + 8;
  static constexpr int TP = D + 32;
};

// ---------------------------------------------------------------- dK, dV ---

template <int DQK, int DV>
struct DkdvCfg {
  static constexpr int BN = 128;      // keys per workgroup
  static constexpr int BMQ = 64;      // queries per step
  static constexpr int NT = 256;
  static constexpr int QNP = TilePitch<DQK>::NP, QTP = TilePitch<DQK>::TP;
  static constexpr int ONP = TilePitch<DV>::NP, OTP = TilePitch<DV>::TP;
  static constexpr int QCH = DQK / 8, OCH = DV / 8;  // 16-byte chunks per row
  static constexpr int QLOADS = BMQ * QCH / NT;
  static constexpr int OLOADS = BMQ * OCH / NT;
  static constexpr int LDS_ELEMS = BMQ * (QNP + QTP + ONP + OTP);
  static_assert(BMQ * QCH % NT == 0 && BMQ * OCH % NT == 0, "tile split");
};

template <int DQK, int DV>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_kernel(KArgs a) {
  using C = DkdvCfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) float lse_s[C::BMQ];
  __shared__ __attribute__((aligned(16))) float delta_s[C::BMQ];
  uint16_t* Qn = lds;                       // [BMQ][QNP] row reads
  uint16_t* Qt = Qn + C::BMQ * C::QNP;      // [BMQ][QTP] transpose loads
  uint16_t* On = Qt + C::BMQ * C::QTP;      // dO, row reads
  uint16_t* Ot = On + C::BMQ * C::ONP;      // dO, transpose loads

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  // Workgroup id -> (key tile, batch, kv head): consecutive ids cover all
  // (batch, kv head) of one key tile, so with B*Hkv a multiple of 8 a given
  // (batch, kv head) always lands on the same XCD and its Q/dO tiles, read
  // again by the neighbouring key tiles, stay in that XCD's L2.  Key tiles in
  // ascending order: under a causal mask the first ones see the most queries.
  const int kt = blockIdx.x / (a.B * a.Hkv);
  const int r = blockIdx.x % (a.B * a.Hkv);
  const int b = r / a.Hkv, g = r % a.Hkv;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  const int j0 = kt * C::BN;
  const int kw0 = j0 + w * 32;
  const int kj = kw0 + l32;
  int qlo_k, qhi_k;  // rows that see this lane's key
  col_query_bounds(m, kj, qlo_k, qhi_k);

  // K^T / V^T operands: lane holds key kj, dims [ks*16 + hf*8, +8); buffer
  // resources end at the valid length, so keys >= L read as zeros.
  bf16x8 kreg[DQK / 16], vreg[DV / 16];
  {
    const size_t kstride = (size_t)a.Hkv * DQK, vstride = (size_t)a.Hkv * DV;
    const __amdgpu_buffer_rsrc_t kres = buf_rsrc(static_cast<const uint16_t*>(a.k) + ((size_t)b * a.S * a.Hkv + g) * DQK,
                                                 (uint32_t)(m.L * kstride * 2));
    const __amdgpu_buffer_rsrc_t vres = buf_rsrc(static_cast<const uint16_t*>(a.v) + ((size_t)b * a.S * a.Hkv + g) * DV,
                                                 (uint32_t)(m.L * vstride * 2));
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks)
      kreg[ks] = as_bf16x8(buf_load16(kres, (uint32_t)(kj * kstride + ks * 16 + hf * 8) * 2));
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
      vreg[ks] = as_bf16x8(buf_load16(vres, (uint32_t)(kj * vstride + ks * 16 + hf * 8) * 2));
  }
  f32x16 dk[DQK / 32], dv[DV / 32];
#pragma unroll
  for (int i = 0; i < DQK / 32; ++i) dk[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < DV / 32; ++i) dv[i] = f32x16{};

  int qlo = 0, qhi = -1;
  if (!query_range(m, j0, j0 + C::BN - 1, qlo, qhi)) { qlo = 0; qhi = -1; }
  const int qs0 = qlo / C::BMQ;
  const int nsteps = qhi < 0 ? 0 : qhi / C::BMQ - qs0 + 1;
  const int total = nsteps * a.G;

  const uint16_t* Qg = static_cast<const uint16_t*>(a.q);
  const uint16_t* dOg = static_cast<const uint16_t*>(a.d_o);
  u32x4 qst[C::QLOADS], ost[C::OLOADS];
  float lse_r = 0.0f, delta_r = 0.0f;
  const size_t qstride = (size_t)a.Hq * DQK, ostride = (size_t)a.Hq * DV;
  auto load_step = [&](int t) {
    const int h = g * a.G + t / nsteps;
    const int q0 = (qs0 + t % nsteps) * C::BMQ;
    const __amdgpu_buffer_rsrc_t qres = buf_rsrc(Qg + ((size_t)b * a.S * a.Hq + h) * DQK, (uint32_t)(m.L * qstride * 2));
    const __amdgpu_buffer_rsrc_t ores = buf_rsrc(dOg + ((size_t)b * a.S * a.Hq + h) * DV, (uint32_t)(m.L * ostride * 2));
#pragma unroll
    for (int rr = 0; rr < C::QLOADS; ++rr) {
      const int c = tid + rr * C::NT, row = c / C::QCH, cc = c % C::QCH;
      qst[rr] = buf_load16(qres, (uint32_t)((q0 + row) * qstride + cc * 8) * 2);
    }
#pragma unroll
    for (int rr = 0; rr < C::OLOADS; ++rr) {
      const int c = tid + rr * C::NT, row = c / C::OCH, cc = c % C::OCH;
      ost[rr] = buf_load16(ores, (uint32_t)((q0 + row) * ostride + cc * 8) * 2);
    }
    if (tid < C::BMQ) {
      const int i = q0 + tid;
      lse_r = i < m.L ? a.lse[((size_t)b * a.Hq + h) * a.S + i] * kLog2e : 0.0f;
    } else if (tid < 2 * C::BMQ) {
      const int i = q0 + tid - C::BMQ;
      delta_r = i < m.L ? a.delta[((size_t)b * a.Hq + h) * a.S + i] : 0.0f;
    }
  };
  auto store_step = [&]() {
#pragma unroll
    for (int rr = 0; rr < C::QLOADS; ++rr) {
      const int c = tid + rr * C::NT, row = c / C::QCH, cc = c % C::QCH;
      *reinterpret_cast<u32x4*>(Qn + row * C::QNP + cc * 8) = qst[rr];
      *reinterpret_cast<u32x4*>(Qt + row * C::QTP + cc * 8) = qst[rr];
    }
#pragma unroll
    for (int rr = 0; rr < C::OLOADS; ++rr) {
      const int c = tid + rr * C::NT, row = c / C::OCH, cc = c % C::OCH;
      *reinterpret_cast<u32x4*>(On + row * C::ONP + cc * 8) = ost[rr];
      *reinterpret_cast<u32x4*>(Ot + row * C::OTP + cc * 8) = ost[rr];
    }
    if (tid < C::BMQ) lse_s[tid] = lse_r;
    else if (tid < 2 * C::BMQ) delta_s[tid - C::BMQ] = delta_r;
  };

  // One 32-query block qb of the staged step, for this wave's 32 keys.
  // Element i of the S / dP accumulators: query q0 + qb*32 + acc_row(i, hf), key kj.
  auto block = [&](int q0, int qb, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks) {
      const bf16x8 qa = as_bf16x8(*reinterpret_cast<const u32x4*>(Qn + (qb * 32 + l32) * C::QNP + ks * 16 + hf * 8));
      s = mfma32(qa, kreg[ks], s);
    }
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks) {
      const bf16x8 oa = as_bf16x8(*reinterpret_cast<const u32x4*>(On + (qb * 32 + l32) * C::ONP + ks * 16 + hf * 8));
      dp = mfma32(oa, vreg[ks], dp);
    }
    const int base = q0 + qb * 32 + hf * 4;
    const int lo_r = qlo_k - base, hi_r = qhi_k - base;
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int ig = 0; ig < 4; ++ig) {
      const int qo = qb * 32 + ig * 8 + hf * 4;
      const f32x4 l4 = *reinterpret_cast<const f32x4*>(lse_s + qo);
      const f32x4 d4 = *reinterpret_cast<const f32x4*>(delta_s + qo);
      float p[4], ds[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = ig * 4 + u;
        float pv = fast_exp2(fmaf(s[i], a.scale_log2, -l4[u]));
        if constexpr (MASKED) {
          const int off = ig * 8 + u;
          pv = (off >= lo_r && off <= hi_r) ? pv : 0.0f;
        }
        p[u] = pv;
        ds[u] = pv * (dp[i] - d4[u]);
      }
      const int slot = ig >> 1, e0 = (ig & 1) * 4;
      pb[slot][e0 + 0] = (__bf16)p[0];
      pb[slot][e0 + 1] = (__bf16)p[1];
      pb[slot][e0 + 2] = (__bf16)p[2];
      pb[slot][e0 + 3] = (__bf16)p[3];
      dsb[slot][e0 + 0] = (__bf16)ds[0];
      dsb[slot][e0 + 1] = (__bf16)ds[1];
      dsb[slot][e0 + 2] = (__bf16)ds[2];
      dsb[slot][e0 + 3] = (__bf16)ds[3];
    }
    // dV^T (dims x keys) += dO^T P ; dK^T (dims x keys) += Q^T dS.
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int db = 0; db < DV / 32; ++db)
        dv[db] = mfma32(lds_tr_operand(Ot, C::OTP, qb * 32 + kk * 16, db * 32, lane), pb[kk], dv[db]);
#pragma unroll
      for (int db = 0; db < DQK / 32; ++db)
        dk[db] = mfma32(lds_tr_operand(Qt, C::QTP, qb * 32 + kk * 16, db * 32, lane), dsb[kk], dk[db]);
    }
  };

  if (total > 0) load_step(0);
  for (int t = 0; t < total; ++t) {
    const int q0 = (qs0 + t % nsteps) * C::BMQ;
    __syncthreads();
    store_step();
    __syncthreads();
    if (t + 1 < total) load_step(t + 1);
#pragma unroll
    for (int qb = 0; qb < C::BMQ / 32; ++qb) {
      const int cls = tile_class(m, q0 + qb * 32, 32, kw0, 32);
      if (cls == TILE_FULL) block(q0, qb, std::false_type{});
      else if (cls == TILE_PARTIAL) block(q0, qb, std::true_type{});
    }
  }

  // Epilogue: lane owns key kj, dims db*32 + acc_row(i, hf).
  if (kj < a.S) {
    uint16_t* dkp = static_cast<uint16_t*>(a.dk) + ((size_t)(b * a.S + kj) * a.Hkv + g) * DQK + hf * 4;
    uint16_t* dvp = static_cast<uint16_t*>(a.dv) + ((size_t)(b * a.S + kj) * a.Hkv + g) * DV + hf * 4;
#pragma unroll
    for (int db = 0; db < DQK / 32; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        u32x2 val = {pack_bf16(dk[db][ig * 4] * a.scale, dk[db][ig * 4 + 1] * a.scale),
                     pack_bf16(dk[db][ig * 4 + 2] * a.scale, dk[db][ig * 4 + 3] * a.scale)};
        *reinterpret_cast<u32x2*>(dkp + db * 32 + ig * 8) = val;
      }
#pragma unroll
    for (int db = 0; db < DV / 32; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        u32x2 val = {pack_bf16(dv[db][ig * 4], dv[db][ig * 4 + 1]),
                     pack_bf16(dv[db][ig * 4 + 2], dv[db][ig * 4 + 3])};
        *reinterpret_cast<u32x2*>(dvp + db * 32 + ig * 8) = val;
      }
  }
}

// -------------------------------------------------------------------- dQ ---

template <int DQK, int DV>
struct DqCfg {
  static constexpr int BM = 128;      // query rows per workgroup
  static constexpr int BN = 64;       // keys per step
  static constexpr int NT = 256;
  static constexpr int KNP = TilePitch<DQK>::NP, KTP = TilePitch<DQK>::TP;
  static constexpr int VNP = TilePitch<DV>::NP;
  static constexpr int KCH = DQK / 8, VCH = DV / 8;
  static constexpr int KLOADS = BN * KCH / NT;
  static constexpr int VLOADS = BN * VCH / NT;
  static constexpr int LDS_ELEMS = BN * (KNP + KTP + VNP);
  static_assert(BN * KCH % NT == 0 && BN * VCH % NT == 0, "tile split");
};

template <int DQK, int DV>
__global__ __launch_bounds__(256, 1) void bwd_dq_bf16_kernel(KArgs a) {
  using C = DqCfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  uint16_t* Kn = lds;                    // [BN][KNP] row reads
  uint16_t* Kt = Kn + C::BN * C::KNP;    // [BN][KTP] transpose loads
  uint16_t* Vn = Kt + C::BN * C::KTP;    // [BN][VNP] row reads

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  // Same tile order as the forward: heavy query tiles first, the heads of a
  // GQA group on consecutive ids kept on one XCD.
  int b, h, qt;
  {
    const int N = a.B * a.Hq * a.n_tiles, chunk = a.G, full = (N / (8 * chunk)) * (8 * chunk);
    int l = blockIdx.x;
    if (l < full) {
      const int xcd = l & 7, slot = l >> 3;
      l = ((slot / chunk) * 8 + xcd) * chunk + slot % chunk;
    }
    const int per_tile = a.B * a.Hq;
    qt = a.n_tiles - 1 - l / per_tile;
    b = (l % per_tile) / a.Hq;
    h = (l % per_tile) % a.Hq;
  }
  const int g = h / a.G;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  const int i0 = qt * C::BM, qw0 = i0 + w * 32, qi = qw0 + l32;
  int klo, khi;
  row_key_bounds(m, qi, klo, khi);

  bf16x8 qreg[DQK / 16], oreg[DV / 16];
  float lse2 = 0.0f, dl = 0.0f;
  {
    const bool ok = qi < m.L;
    const size_t qstride = (size_t)a.Hq * DQK, ostride = (size_t)a.Hq * DV;
    const __amdgpu_buffer_rsrc_t qres = buf_rsrc(static_cast<const uint16_t*>(a.q) + ((size_t)b * a.S * a.Hq + h) * DQK,
                                                 (uint32_t)(m.L * qstride * 2));
    const __amdgpu_buffer_rsrc_t ores = buf_rsrc(static_cast<const uint16_t*>(a.d_o) + ((size_t)b * a.S * a.Hq + h) * DV,
                                                 (uint32_t)(m.L * ostride * 2));
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks)
      qreg[ks] = as_bf16x8(buf_load16(qres, (uint32_t)(qi * qstride + ks * 16 + hf * 8) * 2));
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
      oreg[ks] = as_bf16x8(buf_load16(ores, (uint32_t)(qi * ostride + ks * 16 + hf * 8) * 2));
    if (ok) {
      lse2 = a.lse[((size_t)b * a.Hq + h) * a.S + qi] * kLog2e;
      dl = a.delta[((size_t)b * a.Hq + h) * a.S + qi];
    }
  }
  f32x16 dq[DQK / 32];
#pragma unroll
  for (int i = 0; i < DQK / 32; ++i) dq[i] = f32x16{};

  int lo = 0, hi = -1;
  const int nrow = (i0 + C::BM < m.L ? i0 + C::BM : m.L) - 1;
  if (!key_range(m, i0, nrow, lo, hi)) { lo = 0; hi = -1; }
  const int kt0 = lo / C::BN, kt1 = hi < 0 ? -1 : hi / C::BN;

  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + ((size_t)b * a.S * a.Hkv + g) * DQK;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v) + ((size_t)b * a.S * a.Hkv + g) * DV;
  const size_t kstride = (size_t)a.Hkv * DQK, vstride = (size_t)a.Hkv * DV;
  const __amdgpu_buffer_rsrc_t kres = buf_rsrc(Kg, (uint32_t)(m.L * kstride * 2));
  const __amdgpu_buffer_rsrc_t vres = buf_rsrc(Vg, (uint32_t)(m.L * vstride * 2));
  u32x4 kst[C::KLOADS], vst[C::VLOADS];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int rr = 0; rr < C::KLOADS; ++rr) {
      const int c = tid + rr * C::NT, row = c / C::KCH, cc = c % C::KCH;
      kst[rr] = buf_load16(kres, (uint32_t)((j0 + row) * kstride + cc * 8) * 2);
    }
#pragma unroll
    for (int rr = 0; rr < C::VLOADS; ++rr) {
      const int c = tid + rr * C::NT, row = c / C::VCH, cc = c % C::VCH;
      vst[rr] = buf_load16(vres, (uint32_t)((j0 + row) * vstride + cc * 8) * 2);
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int rr = 0; rr < C::KLOADS; ++rr) {
      const int c = tid + rr * C::NT, row = c / C::KCH, cc = c % C::KCH;
      *reinterpret_cast<u32x4*>(Kn + row * C::KNP + cc * 8) = kst[rr];
      *reinterpret_cast<u32x4*>(Kt + row * C::KTP + cc * 8) = kst[rr];
    }
#pragma unroll
    for (int rr = 0; rr < C::VLOADS; ++rr) {
      const int c = tid + rr * C::NT, row = c / C::VCH, cc = c % C::VCH;
      *reinterpret_cast<u32x4*>(Vn + row * C::VNP + cc * 8) = vst[rr];
    }
  };

  auto tile = [&](int j0, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    f32x16 st[C::BN / 32], dpt[C::BN / 32];
#pragma unroll
    for (int kb = 0; kb < C::BN / 32; ++kb) { st[kb] = f32x16{}; dpt[kb] = f32x16{}; }
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb) {
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(Kn + (kb * 32 + l32) * C::KNP + ks * 16 + hf * 8));
        st[kb] = mfma32(ka, qreg[ks], st[kb]);
      }
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb) {
        const bf16x8 va = as_bf16x8(*reinterpret_cast<const u32x4*>(Vn + (kb * 32 + l32) * C::VNP + ks * 16 + hf * 8));
        dpt[kb] = mfma32(va, oreg[ks], dpt[kb]);
      }
    // Element i of block kb: key j0 + hf*4 + kb*32 + acc_row(i, 0), query qi.
    const int base = j0 + hf * 4;
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
            v2[u] = pv * (dpt[kb][i] - dl);
          }
          t[e] = pack_bf16(v2[0], v2[1]);
        }
        dsb[kb * 2 + half] = as_bf16x8(t);
      }
    // dQ^T (dims x queries) += K^T dS^T
#pragma unroll
    for (int kk = 0; kk < C::BN / 16; ++kk)
#pragma unroll
      for (int db = 0; db < DQK / 32; ++db)
        dq[db] = mfma32(lds_tr_operand(Kt, C::KTP, kk * 16, db * 32, lane), dsb[kk], dq[db]);
  };

  if (kt0 <= kt1) load_tile(kt0 * C::BN);
  for (int kt = kt0; kt <= kt1; ++kt) {
    const int j0 = kt * C::BN;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt < kt1) load_tile(j0 + C::BN);
    const int cls = tile_class(m, qw0, 32, j0, C::BN);
    if (cls == TILE_FULL) tile(j0, std::false_type{});
    else if (cls == TILE_PARTIAL) tile(j0, std::true_type{});
  }

  if (qi < a.S) {
    uint16_t* dqp = static_cast<uint16_t*>(a.dq) + ((size_t)(b * a.S + qi) * a.Hq + h) * DQK + hf * 4;
#pragma unroll
    for (int db = 0; db < DQK / 32; ++db)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        u32x2 val = {pack_bf16(dq[db][ig * 4] * a.scale, dq[db][ig * 4 + 1] * a.scale),
                     pack_bf16(dq[db][ig * 4 + 2] * a.scale, dq[db][ig * 4 + 3] * a.scale)};
        *reinterpret_cast<u32x2*>(dqp + db * 32 + ig * 8) = val;
      }
  }
}

template <int DQK, int DV>
static hipError_t launch_dkdv_cfg(KArgs a, hipStream_t stream) {
  using D = DkdvCfg<DQK, DV>;
  const int nkt = (a.S + D::BN - 1) / D::BN;
  hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<DQK, DV>), dim3((unsigned)(nkt * a.B * a.Hkv)), dim3(D::NT), 0,
                     stream, a);
  return hipGetLastError();
}

template <int DQK, int DV>
static hipError_t launch_dq_cfg(KArgs a, hipStream_t stream) {
  using Q = DqCfg<DQK, DV>;
  a.n_tiles = (a.S + Q::BM - 1) / Q::BM;
  hipLaunchKernelGGL((bwd_dq_bf16_kernel<DQK, DV>), dim3((unsigned)(a.n_tiles * a.B * a.Hq)), dim3(Q::NT), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const KArgs& a, int dqk, int dv, hipStream_t stream) {
  if (dqk == 64 && dv == 64) return launch_dkdv_cfg<64, 64>(a, stream);
  if (dqk == 128 && dv == 128) return launch_dkdv_cfg<128, 128>(a, stream);
  if (dqk == 192 && dv == 128) return launch_dkdv_cfg<192, 128>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq_bf16(const KArgs& a, int dqk, int dv, hipStream_t stream) {
  if (dqk == 64 && dv == 64) return launch_dq_cfg<64, 64>(a, stream);
  if (dqk == 128 && dv == 128) return launch_dq_cfg<128, 128>(a, stream);
  if (dqk == 192 && dv == 128) return launch_dq_cfg<192, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace sdpa
