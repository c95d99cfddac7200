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
// rows (acc_row).  Contractions over the sequence dimension take the
// accumulator-side operand straight from registers and the other operand from
// an LDS copy stored transposed, sequence positions permuted by perm16 to
// match the accumulator's row order.
#include "launch.h"

namespace sdpa {

// ---------------------------------------------------------------- dK, dV ---

template <int DQK, int DV>
struct DkdvCfg {
  static constexpr int BN = 128;      // keys per workgroup
  static constexpr int BMQ = 64;      // queries per step
  static constexpr int NT = 256;
  static constexpr int QP = DQK + 8;  // pitch of row-major Q in LDS
  static constexpr int OP = DV + 8;   // pitch of row-major dO in LDS
  static constexpr int TP = BMQ + 8;  // pitch of transposed Q / dO
  static constexpr int QBLK = (BMQ / 4) * (DQK / 8);  // 4-row x 8-dim blocks
  static constexpr int OBLK = (BMQ / 4) * (DV / 8);
  static constexpr int QLOADS = (QBLK + NT - 1) / NT;
  static constexpr int OLOADS = (OBLK + NT - 1) / NT;
  static constexpr int LDS_ELEMS = BMQ * QP + BMQ * OP + DQK * TP + DV * TP;
};

// Stores a 4-row x 8-dim block both row-major and transposed (permuted rows).
__device__ __forceinline__ void store_block_both(uint16_t* nat, int pitch, uint16_t* tr, int tpitch,
                                                 int row0, int d0, const u32x4 (&x)[4]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) *reinterpret_cast<u32x4*>(nat + (row0 + t) * pitch + d0) = x[t];
  const int pos = perm16(row0);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t x0 = x[0][e], x1 = x[1][e], x2 = x[2][e], x3 = x[3][e];
    u32x2 even = {(x0 & 0xffffu) | (x1 << 16), (x2 & 0xffffu) | (x3 << 16)};
    u32x2 odd = {(x0 >> 16) | (x1 & 0xffff0000u), (x2 >> 16) | (x3 & 0xffff0000u)};
    *reinterpret_cast<u32x2*>(tr + (d0 + 2 * e) * tpitch + pos) = even;
    *reinterpret_cast<u32x2*>(tr + (d0 + 2 * e + 1) * tpitch + pos) = odd;
  }
}

template <int DQK, int DV>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_kernel(KArgs a) {
  using C = DkdvCfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  __shared__ __attribute__((aligned(16))) float lse_s[C::BMQ];
  __shared__ __attribute__((aligned(16))) float delta_s[C::BMQ];
  uint16_t* Qs = lds;
  uint16_t* dOs = Qs + C::BMQ * C::QP;
  uint16_t* Qt = dOs + C::BMQ * C::OP;
  uint16_t* dOt = Qt + DQK * C::TP;

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

  const uint16_t* Kg = static_cast<const uint16_t*>(a.k);
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v);
  // K^T / V^T operands: lane holds key kj, dims [ks*16 + hf*8, +8).
  bf16x8 kreg[DQK / 16], vreg[DV / 16];
  {
    const bool ok = kj < m.L;
    const size_t row = (size_t)(b * a.S + (ok ? kj : 0)) * a.Hkv + g;
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks)
      kreg[ks] = as_bf16x8(ok ? ldg16(Kg + row * DQK + ks * 16 + hf * 8) : u32x4{0, 0, 0, 0});
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
      vreg[ks] = as_bf16x8(ok ? ldg16(Vg + row * DV + ks * 16 + hf * 8) : u32x4{0, 0, 0, 0});
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
  u32x4 qreg_s[C::QLOADS][4], oreg_s[C::OLOADS][4];
  float lse_r = 0.0f, delta_r = 0.0f;
  auto load_step = [&](int t) {
    const int h = g * a.G + t / nsteps;
    const int q0 = (qs0 + t % nsteps) * C::BMQ;
#pragma unroll
    for (int rr = 0; rr < C::QLOADS; ++rr) {
      const int c = tid + rr * C::NT, dg = c % (DQK / 8), rg = c / (DQK / 8);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = q0 + rg * 4 + u;
        qreg_s[rr][u] = (c < C::QBLK && i < m.L)
                            ? ldg16(Qg + ((size_t)(b * a.S + i) * a.Hq + h) * DQK + dg * 8)
                            : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int rr = 0; rr < C::OLOADS; ++rr) {
      const int c = tid + rr * C::NT, dg = c % (DV / 8), rg = c / (DV / 8);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = q0 + rg * 4 + u;
        oreg_s[rr][u] = (c < C::OBLK && i < m.L)
                            ? ldg16(dOg + ((size_t)(b * a.S + i) * a.Hq + h) * DV + dg * 8)
                            : u32x4{0, 0, 0, 0};
      }
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
      const int c = tid + rr * C::NT;
      if (c < C::QBLK) store_block_both(Qs, C::QP, Qt, C::TP, (c / (DQK / 8)) * 4, (c % (DQK / 8)) * 8, qreg_s[rr]);
    }
#pragma unroll
    for (int rr = 0; rr < C::OLOADS; ++rr) {
      const int c = tid + rr * C::NT;
      if (c < C::OBLK) store_block_both(dOs, C::OP, dOt, C::TP, (c / (DV / 8)) * 4, (c % (DV / 8)) * 8, oreg_s[rr]);
    }
    if (tid < C::BMQ) lse_s[tid] = lse_r;
    else if (tid < 2 * C::BMQ) delta_s[tid - C::BMQ] = delta_r;
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
      const int qrow0 = q0 + qb * 32;
      const int cls = tile_class(m, qrow0, 32, kw0, 32);
      if (cls == TILE_SKIP) continue;
      // S and dP (queries x keys): A = Q / dO rows from LDS, B = K^T / V^T regs.
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < DQK / 16; ++ks) {
        const bf16x8 qa = as_bf16x8(*reinterpret_cast<const u32x4*>(Qs + (qb * 32 + l32) * C::QP + ks * 16 + hf * 8));
        s = mfma32(qa, kreg[ks], s);
      }
#pragma unroll
      for (int ks = 0; ks < DV / 16; ++ks) {
        const bf16x8 oa = as_bf16x8(*reinterpret_cast<const u32x4*>(dOs + (qb * 32 + l32) * C::OP + ks * 16 + hf * 8));
        dp = mfma32(oa, vreg[ks], dp);
      }
      // Element i: query qrow0 + acc_row(i, hf), key kj.
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
          float pv = fast_exp2(s[i] * a.scale_log2 - l4[u]);
          if (cls == TILE_PARTIAL && !visible(m, q0 + qo + u, kj)) pv = 0.0f;
          p[u] = pv;
          ds[u] = pv * (dp[i] - d4[u]);
        }
        const int slot = ig >> 1, e0 = (ig & 1) * 2;
        pb[slot][e0 * 2 + 0] = (__bf16)p[0];
        pb[slot][e0 * 2 + 1] = (__bf16)p[1];
        pb[slot][e0 * 2 + 2] = (__bf16)p[2];
        pb[slot][e0 * 2 + 3] = (__bf16)p[3];
        dsb[slot][e0 * 2 + 0] = (__bf16)ds[0];
        dsb[slot][e0 * 2 + 1] = (__bf16)ds[1];
        dsb[slot][e0 * 2 + 2] = (__bf16)ds[2];
        dsb[slot][e0 * 2 + 3] = (__bf16)ds[3];
      }
      // dV^T (dims x keys) += dO^T P ; dK^T (dims x keys) += Q^T dS.
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int db = 0; db < DV / 32; ++db) {
          const bf16x8 oa = as_bf16x8(*reinterpret_cast<const u32x4*>(dOt + (db * 32 + l32) * C::TP + qb * 32 + kk * 16 + hf * 8));
          dv[db] = mfma32(oa, pb[kk], dv[db]);
        }
#pragma unroll
        for (int db = 0; db < DQK / 32; ++db) {
          const bf16x8 qa = as_bf16x8(*reinterpret_cast<const u32x4*>(Qt + (db * 32 + l32) * C::TP + qb * 32 + kk * 16 + hf * 8));
          dk[db] = mfma32(qa, dsb[kk], dk[db]);
        }
      }
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
  static constexpr int KP = DQK + 8;
  static constexpr int VP = DV + 8;
  static constexpr int TP = BN + 8;
  static constexpr int KBLK = (BN / 4) * (DQK / 8);
  static constexpr int KLOADS = (KBLK + NT - 1) / NT;
  static constexpr int VCH = DV / 8;
  static constexpr int VLOADS = BN * VCH / NT;
  static constexpr int LDS_ELEMS = BN * KP + BN * VP + DQK * TP;
  static_assert(BN * VCH % NT == 0, "V tile split");
};

template <int DQK, int DV>
__global__ __launch_bounds__(256, 1) void bwd_dq_bf16_kernel(KArgs a) {
  using C = DqCfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  uint16_t* Ks = lds;
  uint16_t* Vs = Ks + C::BN * C::KP;
  uint16_t* Kt = Vs + C::BN * C::VP;

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

  bf16x8 qreg[DQK / 16], oreg[DV / 16];
  float lse2 = 0.0f, dl = 0.0f;
  {
    const bool ok = qi < m.L;
    const size_t row = (size_t)(b * a.S + (ok ? qi : 0)) * a.Hq + h;
    const uint16_t* Qg = static_cast<const uint16_t*>(a.q);
    const uint16_t* dOg = static_cast<const uint16_t*>(a.d_o);
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks)
      qreg[ks] = as_bf16x8(ok ? ldg16(Qg + row * DQK + ks * 16 + hf * 8) : u32x4{0, 0, 0, 0});
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
      oreg[ks] = as_bf16x8(ok ? ldg16(dOg + row * DV + ks * 16 + hf * 8) : u32x4{0, 0, 0, 0});
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
  u32x4 kreg_s[C::KLOADS][4], vreg_s[C::VLOADS];
  auto load_tile = [&](int j0) {
#pragma unroll
    for (int rr = 0; rr < C::KLOADS; ++rr) {
      const int c = tid + rr * C::NT, dg = c % (DQK / 8), rg = c / (DQK / 8);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + rg * 4 + u;
        kreg_s[rr][u] = (c < C::KBLK && j < m.L) ? ldg16(Kg + (size_t)j * kstride + dg * 8) : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int rr = 0; rr < C::VLOADS; ++rr) {
      const int c = tid + rr * C::NT, row = c / C::VCH, cc = c % C::VCH, j = j0 + row;
      vreg_s[rr] = j < m.L ? ldg16(Vg + (size_t)j * vstride + cc * 8) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int rr = 0; rr < C::KLOADS; ++rr) {
      const int c = tid + rr * C::NT;
      if (c < C::KBLK) store_block_both(Ks, C::KP, Kt, C::TP, (c / (DQK / 8)) * 4, (c % (DQK / 8)) * 8, kreg_s[rr]);
    }
#pragma unroll
    for (int rr = 0; rr < C::VLOADS; ++rr) {
      const int c = tid + rr * C::NT, row = c / C::VCH, cc = c % C::VCH;
      *reinterpret_cast<u32x4*>(Vs + row * C::VP + cc * 8) = vreg_s[rr];
    }
  };

  if (kt0 <= kt1) load_tile(kt0 * C::BN);
  for (int kt = kt0; kt <= kt1; ++kt) {
    const int j0 = kt * C::BN;
    __syncthreads();
    store_tile();
    __syncthreads();
    if (kt < kt1) load_tile(j0 + C::BN);

    const int cls = tile_class(m, qw0, 32, j0, C::BN);
    if (cls == TILE_SKIP) continue;
    f32x16 st[C::BN / 32], dpt[C::BN / 32];
#pragma unroll
    for (int kb = 0; kb < C::BN / 32; ++kb) { st[kb] = f32x16{}; dpt[kb] = f32x16{}; }
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb) {
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(Ks + (kb * 32 + l32) * C::KP + ks * 16 + hf * 8));
        st[kb] = mfma32(ka, qreg[ks], st[kb]);
      }
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb) {
        const bf16x8 va = as_bf16x8(*reinterpret_cast<const u32x4*>(Vs + (kb * 32 + l32) * C::VP + ks * 16 + hf * 8));
        dpt[kb] = mfma32(va, oreg[ks], dpt[kb]);
      }
    // Element i of block kb: key j0 + kb*32 + acc_row(i, hf), query qi.
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
            float pv = fast_exp2(st[kb][i] * a.scale_log2 - lse2);
            if (cls == TILE_PARTIAL && !visible(m, qi, j0 + kb * 32 + acc_row(i, hf))) pv = 0.0f;
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
      for (int db = 0; db < DQK / 32; ++db) {
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4*>(Kt + (db * 32 + l32) * C::TP + kk * 16 + hf * 8));
        dq[db] = mfma32(ka, dsb[kk], dq[db]);
      }
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
