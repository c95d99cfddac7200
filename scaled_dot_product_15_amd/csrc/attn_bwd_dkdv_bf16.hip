// Backward attention, dK and dV, bf16 inputs, fp32 accumulation, gfx950 MFMA 32x32x16.
// Built without the VGPR-form MFMA option: dK and dV accumulate in AGPRs, which
// leaves VGPRs free to keep several LDS reads in flight per MFMA chain.
//
// With P = exp(scale * Q K^T - LSE) recomputed from the forward's LSE and
// delta_i = rowsum(dO * O) from the pre-pass (PR #2225 backward: dz = dO in,
// grad_q, grad_k, grad_v out):
//     dP = dO V^T,  dS = P * (dP - delta),
//     dV = P^T dO,  dK = scale * dS^T Q,  dQ = scale * dS K.
// This kernel (deterministic, no atomics): a workgroup owns BN = 128 keys of
// one (batch, KV head); each wave owns 32 keys and keeps dK, dV in registers
// while the workgroup walks the G query heads of the group in ascending order
// and, for each, the visible query steps in ascending order; the GQA sum is
// therefore a fixed-order register accumulation.  dQ has its own kernel.
// MFMA operand layouts: a lane of a 32x32 accumulator owns one column and 16
// rows (acc_row).  Contractions over head dims read 16-byte row pieces of a
// swizzled row-major LDS tile; contractions over the sequence take the
// accumulator-side operand straight from registers and the other one with
// LDS transpose loads from the same tile (TrReads).  Tiles arrive by
// direct memory-to-LDS copies, double buffered, one barrier per step.
#include <type_traits>

#include "launch.h"

// Tile parameters (build-time overridable for tuning sweeps).
#ifndef SDPA_DKDV_BMQ
#define SDPA_DKDV_BMQ 64
#endif
#ifndef SDPA_DKDV_NQB
#define SDPA_DKDV_NQB 1
#endif

namespace sdpa {

template <int DQK, int DV>
struct DkdvCfg {
  static constexpr int BN = 128;      // keys per workgroup
  static constexpr int BMQ = SDPA_DKDV_BMQ;  // queries per step
  static constexpr int NT = 256;
  static constexpr int QCH = DQK / 8, OCH = DV / 8;  // 16-byte chunks per row
  static constexpr int QT = BMQ * DQK, OT = BMQ * DV;  // elements per tile
  static constexpr int LROWS = BMQ < 64 ? 64 : BMQ;    // lse2 / delta entries staged per step
  static constexpr int STAGE = QT + OT + 2 * LROWS * 2;  // Q, dO, lse2 and delta (f32)
  static constexpr int LDS_ELEMS = 2 * STAGE;
  // 32-query blocks computed together; one at a time keeps registers free
  // for in-flight LDS reads.
  static constexpr int NQB = DQK > 128 ? 1 : SDPA_DKDV_NQB;
};

template <int DQK, int DV>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_kernel(KArgs a) {
  using C = DkdvCfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  // Stage buffer `buf`: Q [BMQ][DQK], dO [BMQ][DV] (swizzled), lse2 [BMQ], delta [BMQ].
  auto qtile = [&](int buf) { return lds + buf * C::STAGE; };
  auto otile = [&](int buf) { return lds + buf * C::STAGE + C::QT; };
  auto lse_s = [&](int buf) { return reinterpret_cast<float*>(lds + buf * C::STAGE + C::QT + C::OT); };
  auto delta_s = [&](int buf) { return lse_s(buf) + C::LROWS; };

  // The wave index is left as a per-lane value here: treated as uniform,
  // it turns the per-block class checks below into scalar branches, and the
  // compiler then keeps far more values live (and spills for 192-dim heads).
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
  const size_t qstride = (size_t)a.Hq * DQK, ostride = (size_t)a.Hq * DV;
  const TileCopy<C::BMQ, C::QCH, C::NT> qcopy(tid, (uint32_t)(qstride * 2));
  const TileCopy<C::BMQ, C::OCH, C::NT> ocopy(tid, (uint32_t)(ostride * 2));
  const RowReads<C::QCH> qrd(lane);
  const RowReads<C::OCH> ord(lane);
  const TrReads<C::QCH> qtr(lane);
  const TrReads<C::OCH> otr(lane);
  auto issue_step = [&](int t, int buf) {
    const int h = g * a.G + t / nsteps;
    const int q0 = (qs0 + t % nsteps) * C::BMQ;
    qcopy.issue(Qg + ((size_t)b * a.S * a.Hq + h) * DQK, (uint32_t)(qstride * 2), q0, m.L, qtile(buf));
    ocopy.issue(dOg + ((size_t)b * a.S * a.Hq + h) * DV, (uint32_t)(ostride * 2), q0, m.L, otile(buf));
    // lse2 and delta rows q0 .. q0+LROWS-1: 64 rows per wave instruction,
    // one 4-byte copy per lane; rows past S arrive as zeros.
    constexpr int PARTS = C::LROWS / 64;
    for (int chunk = w; chunk < 2 * PARTS; chunk += C::NT / 64) {
      const int arr = chunk / PARTS, part = chunk % PARTS;
      const float* src = (arr == 0 ? a.lse2 : a.delta) + ((size_t)b * a.Hq + h) * a.S;
      float* dst = (arr == 0 ? lse_s(buf) : delta_s(buf)) + part * 64;
      lds_dma4(buf_desc(src, (uint32_t)a.S * 4), lds_addr(dst), (uint32_t)(q0 + part * 64 + lane) * 4);
    }
  };

  // NQB consecutive 32-query blocks (from block qb0) of a staged step, for
  // this wave's 32 keys.  Element i of an S / dP accumulator of block qb:
  // query q0 + qb*32 + acc_row(i, hf), key kj.  MASKED evaluates the
  // per-element predicate.
  auto step = [&](int q0, int qb0, int buf, auto masked) {
    constexpr bool MASKED = decltype(masked)::value;
    constexpr int NQB = C::NQB;
    const uint16_t* Qs = qtile(buf);
    const uint16_t* Os = otile(buf);
    const float* ls = lse_s(buf);
    const float* ds_ = delta_s(buf);
    f32x16 s[NQB], dp[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) { s[qb] = f32x16{}; dp[qb] = f32x16{}; }
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        s[qb] = mfma32(as_bf16x8(qrd.read(Qs, (qb0 + qb) * 32, ks)), kreg[ks], s[qb]);
#pragma unroll
    for (int ks = 0; ks < DV / 16; ++ks)
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb)
        dp[qb] = mfma32(as_bf16x8(ord.read(Os, (qb0 + qb) * 32, ks)), vreg[ks], dp[qb]);
    const int lo_r = qlo_k - (q0 + hf * 4), hi_r = qhi_k - (q0 + hf * 4);
    u32x4 pw[2 * NQB], dw[2 * NQB];  // bf16 pairs of P and dS: B operands of the 16-query K-steps
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int qo = (qb0 + qb) * 32 + ig * 8 + hf * 4;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(ls + qo);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(ds_ + qo);
        u32x2 pp, dd;
#pragma unroll
        for (int u2 = 0; u2 < 2; ++u2) {
          float p2[2], s2[2];
#pragma unroll
          for (int v = 0; v < 2; ++v) {
            const int u = u2 * 2 + v, i = ig * 4 + u;
            float pv = fast_exp2(fmaf(s[qb][i], a.scale_log2, -l4[u]));
            if constexpr (MASKED) {
              const int off = (qb0 + qb) * 32 + ig * 8 + u;
              pv = (off >= lo_r && off <= hi_r) ? pv : 0.0f;
            }
            p2[v] = pv;
            s2[v] = pv * (dp[qb][i] - d4[u]);
          }
          pp[u2] = pack_bf16(p2[0], p2[1]);
          dd[u2] = pack_bf16(s2[0], s2[1]);
        }
        // accumulator elements ig*4 .. ig*4+3 of block qb are B-operand
        // elements (ig%2)*4 .. +3 of K-step qb*2 + ig/2
        const int slot = qb * 2 + (ig >> 1), e0 = (ig & 1) * 2;
        pw[slot][e0] = pp[0];
        pw[slot][e0 + 1] = pp[1];
        dw[slot][e0] = dd[0];
        dw[slot][e0 + 1] = dd[1];
      }
    // dV^T (dims x keys) += dO^T P ; dK^T (dims x keys) += Q^T dS.
#pragma unroll
    for (int kk = 0; kk < 2 * NQB; ++kk) {
      const int pos0 = qb0 * 32 + kk * 16;
#pragma unroll
      for (int db = 0; db < DV / 32; ++db)
        dv[db] = mfma32(otr.read(Os, pos0, db), as_bf16x8(pw[kk]), dv[db]);
#pragma unroll
      for (int db = 0; db < DQK / 32; ++db)
        dk[db] = mfma32(qtr.read(Qs, pos0, db), as_bf16x8(dw[kk]), dk[db]);
    }
  };

  // Unrolled by two: each stage's buffer, and so every LDS offset, is a
  // compile-time constant.
  auto stage = [&](int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int q0 = (qs0 + t % nsteps) * C::BMQ;
    if (t + 1 < total) issue_step(t + 1, buf ^ 1);
#pragma unroll
    for (int qb0 = 0; qb0 < C::BMQ / 32; qb0 += C::NQB) {
      bool full = true, any = false;
#pragma unroll
      for (int qb = qb0; qb < qb0 + C::NQB; ++qb) {
        const int cls = tile_class(m, q0 + qb * 32, 32, kw0, 32);
        full = full && cls == TILE_FULL;
        any = any || cls != TILE_SKIP;
      }
      if (full) step(q0, qb0, buf, std::false_type{});
      else if (any) step(q0, qb0, buf, std::true_type{});
    }
    lds_dma_wait();
    __syncthreads();
  };
  if (total > 0) issue_step(0, 0);
  lds_dma_wait();
  __syncthreads();
  for (int t = 0; t < total; t += 2) {
    stage(t, std::integral_constant<int, 0>{});
    if (t + 1 < total) stage(t + 1, std::integral_constant<int, 1>{});
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

// Explicit instantiations: with only the implicit ones from the launchers
// below, the host pass of this compiler drops the launch stub of the last
// kernel instantiated in the file.
template __global__ void bwd_dkdv_bf16_kernel<64, 64>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<128, 128>(KArgs);
template __global__ void bwd_dkdv_bf16_kernel<192, 128>(KArgs);

template <int DQK, int DV>
static hipError_t launch_dkdv_cfg(KArgs a, hipStream_t stream) {
  using D = DkdvCfg<DQK, DV>;
  const int nkt = (a.S + D::BN - 1) / D::BN;
  hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<DQK, DV>), dim3((unsigned)(nkt * a.B * a.Hkv)), dim3(D::NT), 0,
                     stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dkdv_bf16(const KArgs& a, int dqk, int dv, hipStream_t stream) {
  if (dqk == 64 && dv == 64) return launch_dkdv_cfg<64, 64>(a, stream);
  if (dqk == 128 && dv == 128) return launch_dkdv_cfg<128, 128>(a, stream);
  if (dqk == 192 && dv == 128) return launch_dkdv_cfg<192, 128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace sdpa
