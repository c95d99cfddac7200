// Forward attention, bf16 inputs, fp32 accumulation, gfx950 MFMA 32x32x16.
//
// Computes O = softmax(scale * Q K^T + mask [+ sink]) V and the row LSE
// (codelab "Speed up attention on GPU with cuDNN and TransformerEngine",
// "How attention works" steps 1-4, fused into one kernel as its sections 5-6
// describe; sink softmax variants from PR #2225's sequence diagrams).
//
// Work decomposition: one workgroup of 4 waves owns BM = 128 query rows of one
// (batch, query head); each wave owns 32 rows.  The workgroup walks the key
// tiles (BN keys) that the mask engine says are visible from any of its rows,
// all four waves together (one barrier per tile).  Tiles that every row of
// the workgroup sees in full run in an unmasked loop; the others (window
// start, diagonal, padding) run in masked loops that evaluate the predicate
// per element, where a wave whose rows see none of a tile computes it with
// P = 0.
//
// Per key tile and wave:
//   S^T (keys x queries) = K Q^T with A = K rows read from LDS and B = Q^T
//   held in registers for the whole loop.  In the 32x32 accumulator a lane
//   owns one query column, so the row max/sum of the online softmax need a
//   single cross-lane step (lane <-> lane^32).
//   O^T (dims x queries) += V^T P^T with B = P^T taken straight from the S^T
//   accumulator registers (after exp and bf16 rounding) and A = V^T read with
//   LDS transpose loads from the row-major V tile (TrReads).
// K and V tiles reach LDS by direct memory-to-LDS copies into double
// buffers (swizzled rows); K runs two tiles ahead, V one, so the copies are in
// flight while the current tile computes.
//
// Online softmax in base 2 with the scale folded into one FMA.  The running
// max only moves (and O and the row sum are rescaled) when a tile's max
// exceeds it by more than 8, so most tiles skip the rescale; P is then bounded
// by 2^8, harmless in fp32/bf16, and the final O = acc / l and
// LSE = m + log2(l) are exact whichever max was used.  A sink logit z starts
// the running max at z with row sum 1 (its own exp term).
//
// DROP (attention dropout): the P tile fed to P V keeps a probability only
// where the pair's random byte passes the threshold (dropout.h); the row sum
// takes every probability, and O is scaled by 1 / (1 - p) in the epilogue.
//
// BIAS (additive post-scale attention bias, s = scale q.k + bias): bias / scale
// is added to the unscaled scores of each tile before its max; each lane
// loads its row's 64 bias values of the next tile while the current one
// computes (RowBias).
#include <type_traits>

#include "attn_common.h"
#include "dropout.h"
#include "launch.h"

// Tile parameters (build-time overridable for tuning sweeps).
#ifndef SDPA_FWD_BN
#define SDPA_FWD_BN 64
#endif
#ifndef SDPA_FWD_WAVES
#define SDPA_FWD_WAVES 4
#endif

namespace sdpa {

template <int DQK, int DV, int BN>
struct FwdBf16Cfg {
  static constexpr int BM = 32 * SDPA_FWD_WAVES;  // query rows per workgroup (32 per wave)
  static constexpr int NT = 64 * SDPA_FWD_WAVES;
  static constexpr int KCH = DQK / 8;   // 16-byte chunks per K row
  static constexpr int VCH = DV / 8;
  static constexpr int KT = BN * DQK;   // elements of one K tile
  static constexpr int VT = BN * DV;
  static constexpr int LDS_ELEMS = 2 * (KT + VT);  // double buffered
  static_assert(BN % 32 == 0 && DQK % 32 == 0 && DV % 32 == 0, "tile shape");
};

template <int DQK, int DV, int BN, int OCC, bool DROP, bool BIAS>
__global__ __launch_bounds__(64 * SDPA_FWD_WAVES, OCC) void fwd_bf16_kernel(KArgs a) {
  using C = FwdBf16Cfg<DQK, DV, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];

  const int tid = threadIdx.x, w = wave_id(tid), lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  int b, h, qt;
  q_tile_of<kGroupedOrder<DQK>>(a, blockIdx.x, b, h, qt);
  const int g = h / a.G;
  const int bh = b * a.Hq + h;
  const DropGen dg = drop_gen(a);
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  const int i0 = qt * C::BM;
  const int row_w0 = i0 + w * 32;
  const int qi = row_w0 + l32;
  int klo, khi;  // keys visible from this lane's query row
  row_key_bounds(m, qi, klo, khi);

  const uint16_t* Q = static_cast<const uint16_t*>(a.q);
  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + (seq_row0(a, b) * a.Hkv + g) * DQK;
  const uint16_t* Vg = static_cast<const uint16_t*>(a.v) + (seq_row0(a, b) * a.Hkv + g) * DV;
  const size_t kstride = (size_t)a.Hkv * DQK, vstride = (size_t)a.Hkv * DV;

  const TileCopy<BN, C::KCH, C::NT> kcopy(tid, (uint32_t)(kstride * 2));
  const TileCopy<BN, C::VCH, C::NT> vcopy(tid, (uint32_t)(vstride * 2));
  const RowReads<C::KCH> krd(lane);
  const TrReads<C::VCH> vrd(lane);

  // Q^T operand: lane holds query qi, dims [ks*16 + hf*8, +8).
  bf16x8 qreg[DQK / 16];
  {
    const size_t qstride = (size_t)a.Hq * DQK;
    const __amdgpu_buffer_rsrc_t qres = buf_rsrc(Q + (seq_row0(a, b) * a.Hq + h) * DQK, (uint32_t)(m.L * qstride * 2));
    const uint32_t qoff = (uint32_t)(qi * qstride + hf * 8) * 2;
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks) qreg[ks] = as_bf16x8(buf_load16(qres, qoff + ks * 32));
  }

  const float c = a.scale_log2;  // > 0
  const float z2 = sink_logit(a, h) * kLog2e;
  const bool has_sink = a.softmax_type != 0;
  float m_run = has_sink ? z2 : -__builtin_inff();
  float l_run = (has_sink && hf == 0) ? 1.0f : 0.0f;
  f32x16 o[DV / 32];
#pragma unroll
  for (int db = 0; db < DV / 32; ++db) o[db] = f32x16{};

  int lo = 0, hi = -1;
  const int nrow = (i0 + C::BM < m.L ? i0 + C::BM : m.L) - 1;
  if (!key_range(m, i0, nrow, lo, hi)) { lo = 0; hi = -1; }
  const int kt0 = lo / BN, kt1 = hi < 0 ? -1 : hi / BN;
  RowBias<BN / 32> bias;
  if constexpr (BIAS) bias.init(a, b, h, qi, hf);

  // K / V tiles of buffer `buf`: [BN][DQK] and [BN][DV], swizzled row-major.
  auto ktile = [&](int buf) __attribute__((always_inline)) { return lds + buf * (C::KT + C::VT); };
  auto vtile = [&](int buf) __attribute__((always_inline)) { return lds + buf * (C::KT + C::VT) + C::KT; };

  // Software pipeline over key tiles: iteration k finishes tile k (mask,
  // online softmax, P V) and computes the scores of tile k+1, so the score
  // products of k+1 and the exp / pack work of k sit in one basic block and
  // overlap.  K and V have separate double buffers: at the start of
  // iteration k the copies of K(k+2) (into the slot S(k) was read from) and
  // V(k+1) (into the slot P V(k-1) read) are issued; both land before the
  // barrier that closes the iteration.  The scores of the tile after the
  // last one are computed from whatever the slot holds and never used.
  f32x16 sc[2][BN / 32];  // scores of tile k (slot k&1) and of tile k+1
  auto scores = [&](const uint16_t* Ks, f32x16 (&s)[BN / 32]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < DQK / 16; ++ks) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        const bf16x8 ka = as_bf16x8(krd.read(Ks, kb * 32, ks));
        s[kb] = mfma32(ka, qreg[ks], s[kb]);
      }
    }
  };
  // MASKED selects the per-element predicate: element i of block kb of tile
  // k is key j0 + hf*4 + kb*32 + acc_row(i, 0).
  auto iteration = [&](int kt, auto bufc, auto masked) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    constexpr bool MASKED = decltype(masked)::value;
    const int j0 = kt * BN;
    if (kt + 2 <= kt1) kcopy.issue(Kg, (uint32_t)(kstride * 2), j0 + 2 * BN, m.L, ktile(buf));
    if (kt + 1 <= kt1) vcopy.issue(Vg, (uint32_t)(vstride * 2), j0 + BN, m.L, vtile(buf ^ 1));
    f32x16 (&s)[BN / 32] = sc[buf];
    if constexpr (BIAS) {
      bias.add(s, a.inv_scale);            // tile kt's bias, loaded one iteration ago
      if (kt + 1 <= kt1) bias.load(j0 + BN);  // lands by the barrier closing this iteration
    }
    float mx = -__builtin_inff();
    if constexpr (MASKED) {
      const int base = j0 + hf * 4;
      const int lo_r = klo - base, hi_r = khi - base;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = kb * 32 + (i >> 2) * 8 + (i & 3);
          s[kb][i] = (off >= lo_r && off <= hi_r) ? s[kb][i] : -__builtin_inff();
        }
    }
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
    mx = halves_max(mx) * c;
    const float m_new = fmaxf(m_run, mx);
    const bool rescale = __any(m_new > m_run + 8.0f);
    if (__builtin_expect(rescale, 0)) {
      const float alpha = (m_new == -__builtin_inff()) ? 1.0f : fast_exp2(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DV / 32; ++db) o[db] *= alpha;
    }
    const float nmu = (m_run == -__builtin_inff()) ? 0.0f : -m_run;
    // From here to the barrier one basic block: the scores of the next tile
    // (issued first so the matrix unit starts while the exp work below
    // runs), this tile's exp / pack, and its P V products.
    scores(ktile(buf ^ 1), sc[buf ^ 1]);
    // Dropout: random bytes of keys j0 + kb*32 + g*8 + hf*4 + 0..3 (the
    // accumulator elements 4g .. 4g+3 of block kb) for this lane's row.
    uint32_t rnd[BN / 32][4];
    if constexpr (DROP) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) drop_rows_quad(dg, bh, qi, j0 + kb * 32 + hf * 4, rnd[kb]);
    }
    float ls = 0.0f;
    bf16x8 pb[BN / 16];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        u32x4 t;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float p0 = fast_exp2(fmaf(s[kb][half * 8 + 2 * e], c, nmu));
          float p1 = fast_exp2(fmaf(s[kb][half * 8 + 2 * e + 1], c, nmu));
          ls += p0 + p1;
          if constexpr (DROP) {
            // elements half*8 + 2e, +1: group half*2 + e/2, bytes (2e) % 4, +1
            const uint32_t r4 = rnd[kb][half * 2 + (e >> 1)];
            p0 = drop_keep(r4, (2 * e) & 3, dg.t) ? p0 : 0.0f;
            p1 = drop_keep(r4, ((2 * e) & 3) + 1, dg.t) ? p1 : 0.0f;
          }
          t[e] = pack_bf16(p0, p1);
        }
        pb[kb * 2 + half] = as_bf16x8(t);
      }
    }
    l_run += ls;
    const uint16_t* Vs = vtile(buf);
#pragma unroll
    for (int kk = 0; kk < BN / 16; ++kk) {
#pragma unroll
      for (int db = 0; db < DV / 32; ++db) {
        const bf16x8 va = vrd.read(Vs, kk * 16, db);
        o[db] = mfma32(va, pb[kk], o[db]);
      }
    }
    lds_dma_wait();
    __syncthreads();
  };

  // Key tiles that every row of the workgroup sees in full run unmasked; the
  // rest (window start, diagonal, padding) run with the mask (a wave whose
  // rows see none of a tile gets P = 0 there).  Tiles go in pairs (slots 0,
  // 1) so every LDS offset is a compile-time constant; the unmasked range is
  // trimmed to whole pairs, and each of the three loops has a single code
  // path so the accumulators stay in place.
  int fa = kt0, fb = kt0;  // unmasked tiles [fa, fb); fa - kt0, fb - fa even
  {
    int f0, f1;
    if (kt0 <= kt1 && full_key_tiles(m, i0, C::BM, BN, f0, f1)) {
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
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  // Tile slots follow k - kt0; tile k0 = kt0 lands in slot 0.
  if (kt0 <= kt1) {
    kcopy.issue(Kg, (uint32_t)(kstride * 2), kt0 * BN, m.L, ktile(0));
    vcopy.issue(Vg, (uint32_t)(vstride * 2), kt0 * BN, m.L, vtile(0));
    if (kt0 + 1 <= kt1) kcopy.issue(Kg, (uint32_t)(kstride * 2), (kt0 + 1) * BN, m.L, ktile(1));
    if constexpr (BIAS) bias.load(kt0 * BN);
    lds_dma_wait();
    __syncthreads();
    prio_mfma();
    scores(ktile(0), sc[0]);
    prio_valu();
  }
  for (int kt = kt0; kt < fa; kt += 2) {
    iteration(kt, B0{}, std::true_type{});
    iteration(kt + 1, B1{}, std::true_type{});
  }
  for (int kt = fa; kt < fb; kt += 2) {
    iteration(kt, B0{}, std::false_type{});
    iteration(kt + 1, B1{}, std::false_type{});
  }
  for (int kt = fb; kt <= kt1; kt += 2) {
    iteration(kt, B0{}, std::true_type{});
    if (kt + 1 <= kt1) iteration(kt + 1, B1{}, std::true_type{});
  }

  // Epilogue: O = acc / l, LSE = (m + log2 l) * ln 2.
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.0f ? (DROP ? dg.scale : 1.0f) / l_tot : 0.0f;
  // O rows exist up to the batch's row count (S, or the segment size of
  // packed tensors); LSE rows up to S.
  if (qi < seq_rows(a, b)) {
    uint16_t* op = static_cast<uint16_t*>(a.out_o) + ((seq_row0(a, b) + qi) * a.Hq + h) * DV + hf * 4;
#pragma unroll
    for (int db = 0; db < DV / 32; ++db) {
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        u32x2 val = {pack_bf16(o[db][ig * 4] * inv, o[db][ig * 4 + 1] * inv),
                     pack_bf16(o[db][ig * 4 + 2] * inv, o[db][ig * 4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + db * 32 + ig * 8) = val;
      }
    }
  }
  if (qi < a.S) {
    if (hf == 0) {
      const float lse2 = l_tot > 0.0f ? m_run + __log2f(l_tot) : -__builtin_inff();
      a.out_lse[((size_t)b * a.Hq + h) * a.S + qi] = lse2 * kLn2;
    }
  }
}

// Occupancy (workgroups per CU) each head-dim configuration is built for.
constexpr int kFwdOcc64 = SDPA_FWD_WAVES > 4 ? 1 : 2;
constexpr int kFwdOcc128 = (SDPA_FWD_BN > 64 || SDPA_FWD_WAVES > 4) ? 1 : 2;
constexpr int kFwdOcc192 = 1;

// Explicit instantiations: with only the implicit ones from the launchers
// below, the host pass of this compiler drops the launch stub of the last
// kernel instantiated in the file.
// The dropout variants are built with a one-workgroup bound so the
// generator's state can never force spills; at head dims up to 128 they still
// fit the two-workgroup register budget and run two per CU.
template __global__ void fwd_bf16_kernel<64, 64, SDPA_FWD_BN, kFwdOcc64, false, false>(KArgs);
template __global__ void fwd_bf16_kernel<128, 128, SDPA_FWD_BN, kFwdOcc128, false, false>(KArgs);
template __global__ void fwd_bf16_kernel<192, 128, SDPA_FWD_BN, kFwdOcc192, false, false>(KArgs);
template __global__ void fwd_bf16_kernel<64, 64, SDPA_FWD_BN, 1, true, false>(KArgs);
template __global__ void fwd_bf16_kernel<128, 128, SDPA_FWD_BN, 1, true, false>(KArgs);
template __global__ void fwd_bf16_kernel<192, 128, SDPA_FWD_BN, 1, true, false>(KArgs);
// Bias variants (head dims 64 and 128), with the same one-workgroup bound.
template __global__ void fwd_bf16_kernel<64, 64, SDPA_FWD_BN, 1, false, true>(KArgs);
template __global__ void fwd_bf16_kernel<128, 128, SDPA_FWD_BN, 1, false, true>(KArgs);
template __global__ void fwd_bf16_kernel<64, 64, SDPA_FWD_BN, 1, true, true>(KArgs);
template __global__ void fwd_bf16_kernel<128, 128, SDPA_FWD_BN, 1, true, true>(KArgs);

template <int DQK, int DV, int BN, int OCC>
static hipError_t launch_fwd_cfg(KArgs a, hipStream_t stream) {
  using C = FwdBf16Cfg<DQK, DV, BN>;
  a.n_tiles = (a.S + C::BM - 1) / C::BM;
  const long long n = (long long)a.B * a.Hq * a.n_tiles;
  const dim3 grid((unsigned)n), block(C::NT);
  if constexpr (DQK <= 128) {
    if (a.bias) {
      if (a.drop_t > 0) hipLaunchKernelGGL((fwd_bf16_kernel<DQK, DV, BN, 1, true, true>), grid, block, 0, stream, a);
      else hipLaunchKernelGGL((fwd_bf16_kernel<DQK, DV, BN, 1, false, true>), grid, block, 0, stream, a);
      return hipGetLastError();
    }
  } else if (a.bias) {
    return hipErrorInvalidValue;  // no bias variant for these head dims
  }
  if (a.drop_t > 0) hipLaunchKernelGGL((fwd_bf16_kernel<DQK, DV, BN, 1, true, false>), grid, block, 0, stream, a);
  else hipLaunchKernelGGL((fwd_bf16_kernel<DQK, DV, BN, OCC, false, false>), grid, block, 0, stream, a);
  return hipGetLastError();
}

bool fwd_bf16_tiles(int dqk, int dv, int* bm, int* bn) {
  const bool ok = (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
  if (ok) {
    *bm = 32 * SDPA_FWD_WAVES;
    *bn = SDPA_FWD_BN;
  }
  return ok;
}

hipError_t launch_fwd_bf16(const KArgs& a, int dqk, int dv, hipStream_t stream) {
  constexpr int BN = SDPA_FWD_BN;
  if (dqk == 64 && dv == 64) return launch_fwd_cfg<64, 64, BN, kFwdOcc64>(a, stream);
  if (dqk == 128 && dv == 128) return launch_fwd_cfg<128, 128, BN, kFwdOcc128>(a, stream);
  if (dqk == 192 && dv == 128) return launch_fwd_cfg<192, 128, BN, kFwdOcc192>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace sdpa
