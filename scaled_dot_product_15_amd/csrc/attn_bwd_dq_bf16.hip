// Backward attention (dQ), bf16 inputs, fp32 accumulation, gfx950 MFMA 32x32x16.
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
// rows (acc_row).  Contractions over head dims read 16-byte row pieces of a
// swizzled row-major LDS tile; contractions over the sequence take the
// accumulator-side operand straight from registers and the other one with
// LDS transpose loads from the same tile (tile_tr_operand).  Tiles arrive by
// direct memory-to-LDS copies, double buffered, one barrier per step.
#include <type_traits>

#include "launch.h"

namespace sdpa {

// -------------------------------------------------------------------- dQ ---

template <int DQK, int DV>
struct DqCfg {
  static constexpr int BM = 128;      // query rows per workgroup
  static constexpr int BN = 64;       // keys per step
  static constexpr int NT = 256;
  static constexpr int KCH = DQK / 8, VCH = DV / 8;
  static constexpr int KT = BN * DQK, VT = BN * DV;
  static constexpr int LDS_ELEMS = 2 * (KT + VT);
};

template <int DQK, int DV>
__global__ __launch_bounds__(256, 1) void bwd_dq_bf16_kernel(KArgs a) {
  using C = DqCfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  auto ktile = [&](int buf) { return lds + buf * (C::KT + C::VT); };
  auto vtile = [&](int buf) { return lds + buf * (C::KT + C::VT) + C::KT; };

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
    if (qi < m.L) {
      lse2 = a.lse2[((size_t)b * a.Hq + h) * a.S + qi];
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
  auto issue_tile = [&](int j0, int buf) {
    tile_dma<C::BN, C::KCH, C::NT>(kres, (uint32_t)(kstride * 2), j0, ktile(buf), tid);
    tile_dma<C::BN, C::VCH, C::NT>(vres, (uint32_t)(vstride * 2), j0, vtile(buf), tid);
  };

  auto tile = [&](int j0, const uint16_t* Ks, const uint16_t* Vs, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    f32x16 st[C::BN / 32], dpt[C::BN / 32];
#pragma unroll
    for (int kb = 0; kb < C::BN / 32; ++kb) { st[kb] = f32x16{}; dpt[kb] = f32x16{}; }
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb)
        st[kb] = mfma32(as_bf16x8(tile_row16<C::KCH>(Ks, kb * 32 + l32, ks * 2 + hf)), qreg[ks], st[kb]);
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb)
        dpt[kb] = mfma32(as_bf16x8(tile_row16<C::VCH>(Vs, kb * 32 + l32, ks * 2 + hf)), oreg[ks], dpt[kb]);
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
        dq[db] = mfma32(tile_tr_operand<C::KCH>(Ks, kk * 16, db * 32, lane), dsb[kk], dq[db]);
  };

  if (kt0 <= kt1) issue_tile(kt0 * C::BN, 0);
  lds_dma_wait();
  __syncthreads();
  for (int kt = kt0; kt <= kt1; ++kt) {
    const int j0 = kt * C::BN, buf = (kt - kt0) & 1;
    if (kt < kt1) issue_tile(j0 + C::BN, buf ^ 1);
    const int cls = tile_class(m, qw0, 32, j0, C::BN);
    if (cls == TILE_FULL) tile(j0, ktile(buf), vtile(buf), std::false_type{});
    else if (cls == TILE_PARTIAL) tile(j0, ktile(buf), vtile(buf), std::true_type{});
    lds_dma_wait();
    __syncthreads();
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
static hipError_t launch_dq_cfg(KArgs a, hipStream_t stream) {
  using Q = DqCfg<DQK, DV>;
  a.n_tiles = (a.S + Q::BM - 1) / Q::BM;
  hipLaunchKernelGGL((bwd_dq_bf16_kernel<DQK, DV>), dim3((unsigned)(a.n_tiles * a.B * a.Hq)), dim3(Q::NT), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dq_bf16(const KArgs& a, int dqk, int dv, hipStream_t stream) {
  if (dqk == 64 && dv == 64) return launch_dq_cfg<64, 64>(a, stream);
  if (dqk == 128 && dv == 128) return launch_dq_cfg<128, 128>(a, stream);
  if (dqk == 192 && dv == 128) return launch_dq_cfg<192, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace sdpa
