// Backward attention, dQ from stored dS, bf16, fp32 accumulation, gfx950
// MFMA 32x32x16.
//
// dQ = scale * dS K (PR #2225 backward: grad_q; dS = P * (dP - delta) as in
// the other backward kernels).  When the workspace holds the bf16 dS blocks
// the dK/dV kernel wrote (the B operands of its dK products: -dS without
// dropout, where that kernel starts the dP accumulator at delta and negates
// V, dS with it; ds_stored_sign), dQ is a
// contraction of those blocks with K, with no recomputation of S or dP; the
// pass is bound by streaming the blocks from HBM.  Deterministic: each
// workgroup owns its rows' dQ and adds the key tiles in ascending order.
//
// Work decomposition: one workgroup of 4 waves owns 256 query rows of one
// (batch, query head), 64 per wave (two 32-row blocks, so each K^T operand
// read from LDS feeds two products), and walks the visible keys in steps of
// 32 (a quarter of a dK/dV key tile).  Per step, direct memory-to-LDS copies
// bring the K rows ([32][DQK], swizzled) and each block's dS ([32 keys][32
// positions], swizzled 64-byte rows) into a ring of LDS slots, one barrier
// per step.  The pass waits on its copies (the products are short), so the
// ring is as deep as two workgroups per CU allow: three slots, copies two
// steps ahead, up to head dim 128; two at 192.  Workgroups run in the
// forward's order (q_tile_of): from head dim 128 up, a KV head's query tiles
// run together on one XCD and share its K tiles through that XCD's L2.
//
// Layouts.  In a stored block a lane of the dK/dV kernel holds key c = l % 32
// and the 16 rows acc_row(i, l / 32), i = 0..15, of a 32-row block; here
// those are positions p = (l / 32) * 16 + i of key c's 64-byte row.  The
// contraction runs over keys, so both operands come from LDS transpose loads
// (TrReads), which hand a lane the same 8 keys of each 16-key step:
//     dQ^T (dims x positions) += K^T (dims x keys) dS^T (keys x positions).
// Accumulator element i of dim block db, lane l: dim db*32 + acc_row(i, l/32),
// position p = l % 32, i.e. row acc_row(p % 16, p / 16) of the block.
#include <type_traits>

#include "launch.h"

namespace sdpa {

template <int DQK>
struct DqDsCfg {
  static constexpr int BM = 256;         // query rows per workgroup (64 per wave)
  static constexpr int BK = 32;          // keys per step
  static constexpr int NT = 256;
  static constexpr int KCH = DQK / 8;    // 16-byte chunks per K row
  static constexpr int KT = BK * DQK;    // K tile elements
  static constexpr int DT = BK * 32;     // one block's dS tile elements
  static constexpr int STAGE = KT + 8 * DT;
  static constexpr int NSLOT = DQK <= 128 ? 3 : 2;  // ring slots (copies NSLOT - 1 steps ahead)
  static constexpr int LDS_ELEMS = NSLOT * STAGE;
  // Copy instructions per wave and step: the K tile's share and two dS blocks.
  static constexpr int COPIES = BK * KCH / NT + 4;
};

// s_waitcnt with vmcnt = n (< 64), expcnt and lgkmcnt at their no-wait maxima.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int DQK>
__global__ __launch_bounds__(256, 2) void bwd_dq_ds_bf16_kernel(KArgs a) {
  using C = DqDsCfg<DQK>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  auto ktile = [&](int buf) __attribute__((always_inline)) { return lds + buf * C::STAGE; };
  // dS tile of row block rb (0, 1) of wave wv
  auto dtile = [&](int buf, int wv, int rb) __attribute__((always_inline)) {
    return lds + buf * C::STAGE + C::KT + (wv * 2 + rb) * C::DT;
  };

  const int tid = threadIdx.x, w = wave_id(tid), lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  int b, h, qt;
  q_tile_of<kGroupedOrder<DQK>>(a, blockIdx.x, b, h, qt);
  const int g = h / a.G;
  const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
  const int i0 = qt * C::BM, qw0 = i0 + w * 64;

  f32x16 dq[2][DQK / 32];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int i = 0; i < DQK / 32; ++i) dq[rb][i] = f32x16{};

  int lo = 0, hi = -1;
  const int nrow = (i0 + C::BM < m.L ? i0 + C::BM : m.L) - 1;
  if (!key_range(m, i0, nrow, lo, hi)) { lo = 0; hi = -1; }
  const int s0 = lo / C::BK, s1 = hi < 0 ? -1 : hi / C::BK;

  const uint16_t* Kg = static_cast<const uint16_t*>(a.k) + (seq_row0(a, b) * a.Hkv + g) * DQK;
  const size_t kstride = (size_t)a.Hkv * DQK;
  const TileCopy<C::BK, C::KCH, C::NT> kcopy(tid, (uint32_t)(kstride * 2));
  static_assert(TileCopy<C::BK, C::KCH, C::NT>::PER_WAVE + 4 == C::COPIES, "copy count");
  const TrReads<C::KCH> ktr(lane);
  const TrReads<4> dtr(lane);
  // dS copy of one block: two 64-lane instructions; lane l of instruction k
  // fills physical chunk k*64 + l, i.e. key row (k*64+l)/4, logical chunk
  // ch = slot ^ swz<4>(row): positions 8ch .. 8ch+7, which are 16 bytes of
  // the stored lane row + 32 (ch / 2).
  uint32_t dvoff[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int idx = k * 64 + lane, row = idx >> 2, ch = (idx & 3) ^ swz<4>(row);
    dvoff[k] = (uint32_t)((row + 32 * (ch >> 1)) * 32 + (ch & 1) * 16);
  }
  const uint16_t* dsh = a.ds + (size_t)(b * a.Hq + h) * a.ds_head_blocks * 4096;
  // Slab of the key tile being copied (ds_slab), advanced tile by tile as
  // the steps ascend.
  const MaskSpec mf = make_mask(a.S, a.S, a.causal, a.wl, a.wr);
  int sl_kt = s0 >> 2, sl_first, sl_count;
  ds_slab(a, sl_kt, sl_first, sl_count);
  // Copies of step st into slot buf; steps past s1 copy nothing (empty
  // resources land zeros) but keep the per-step instruction count, so the
  // waits below count whole steps.
  auto issue_step = [&](int st, int buf) __attribute__((always_inline)) {
    const int j0 = st * C::BK;
    const bool live = st <= s1;
    kcopy.issue(Kg, (uint32_t)(kstride * 2), j0, live ? m.L : 0, ktile(buf));
    // Each row block's block in the slab of key tile kt = st / 4: rows from
    // q_first, the tile's first visible row rounded down to 64, for 2 nsteps
    // blocks at this batch's length; its 32-key group st % 4.  Groups no row
    // of the block sees were not stored (tile_class SKIP), nor were blocks
    // outside that range: those are not read (empty resource: zeros).
    const int kt = st >> 2;
    while (sl_kt < kt) {
      sl_first += sl_count;
      sl_count = ds_tile_blocks(mf, ++sl_kt);
    }
    int qlo, qhi;
    int r0 = -1, nblk = 0;
    if (live && query_range(m, kt * 128, kt * 128 + 127, qlo, qhi)) {
      nblk = 2 * (qhi / 64 - qlo / 64 + 1);
      if (nblk > sl_count) nblk = sl_count;
      r0 = (qw0 - (qlo / 64) * 64) >> 5;
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int r = r0 + rb;
      const bool ok = r >= 0 && r < nblk && tile_class(m, qw0 + rb * 32, 32, j0, C::BK) != TILE_SKIP;
      const uint16_t* src = dsh + ((size_t)sl_first + (ok ? r : 0)) * 4096 + (st & 3) * 1024;
      const BufDesc d = buf_desc(src, ok ? 2048u : 0u);
      const uint32_t dst = lds_addr(dtile(buf, w, rb));
#pragma unroll
      for (int k = 0; k < 2; ++k) lds_dma16_nt(d, dst + k * 1024, dvoff[k]);
    }
  };
  // Step st from slot buf: wait for its copies (those of the NSLOT - 2 later
  // steps may still be in flight; only these copies are outstanding in the
  // loop, and loads complete in order), barrier, refill the slot read in the
  // previous step with step st + NSLOT - 1, then the products.
  auto step = [&](int st, auto bufc) __attribute__((always_inline)) {
    constexpr int buf = decltype(bufc)::value;
    wait_vmcnt<(C::NSLOT - 2) * C::COPIES>();
    __syncthreads();
    issue_step(st + C::NSLOT - 1, (buf + C::NSLOT - 1) % C::NSLOT);
    // Blocks whose rows see none of the step's keys hold zeros: a step that
    // neither block of the wave sees is skipped.
    const int j0 = st * C::BK;
    if (tile_class(m, qw0, 32, j0, C::BK) != TILE_SKIP || tile_class(m, qw0 + 32, 32, j0, C::BK) != TILE_SKIP) {
#pragma unroll
      for (int t = 0; t < C::BK / 16; ++t) {
        const bf16x8 ds0 = dtr.read(dtile(buf, w, 0), t * 16, 0);
        const bf16x8 ds1 = dtr.read(dtile(buf, w, 1), t * 16, 0);
#pragma unroll
        for (int db = 0; db < DQK / 32; ++db) {
          const bf16x8 kop = ktr.read(ktile(buf), t * 16, db);
          dq[0][db] = mfma32(kop, ds0, dq[0][db]);
          dq[1][db] = mfma32(kop, ds1, dq[1][db]);
        }
      }
    }
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  using B2 = std::integral_constant<int, 2>;
  if (s0 <= s1) {
#pragma unroll
    for (int k = 0; k < C::NSLOT - 1; ++k) issue_step(s0 + k, k);
    if constexpr (C::NSLOT == 3) {
      for (int st = s0; st <= s1; st += 3) {
        step(st, B0{});
        if (st + 1 <= s1) step(st + 1, B1{});
        if (st + 2 <= s1) step(st + 2, B2{});
      }
    } else {
      for (int st = s0; st <= s1; st += 2) {
        step(st, B0{});
        if (st + 1 <= s1) step(st + 1, B1{});
      }
    }
  }
  // Copies of the steps past s1 may still be in flight: wait before the
  // workgroup's LDS can pass to another one.
  lds_dma_wait();

  // Lane: position l32 -> row acc_row(l32 % 16, l32 / 16) of each block;
  // dims db*32 + ig*8 + hf*4 + 0..3 from elements 4 ig .. 4 ig + 3.  The
  // blocks hold dS times ds_stored_sign, so dQ = sign * scale * acc.
  const float qs = ds_stored_sign(a) * a.scale;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int qi = qw0 + rb * 32 + acc_row(l32 & 15, l32 >> 4);
    if (qi < seq_rows(a, b)) {
      uint16_t* dqp = static_cast<uint16_t*>(a.dq) + ((seq_row0(a, b) + qi) * a.Hq + h) * DQK + hf * 4;
#pragma unroll
      for (int db = 0; db < DQK / 32; ++db)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          u32x2 val = {pack_bf16(dq[rb][db][ig * 4] * qs, dq[rb][db][ig * 4 + 1] * qs),
                       pack_bf16(dq[rb][db][ig * 4 + 2] * qs, dq[rb][db][ig * 4 + 3] * qs)};
          *reinterpret_cast<u32x2*>(dqp + db * 32 + ig * 8) = val;
        }
    }
  }
}

template __global__ void bwd_dq_ds_bf16_kernel<64>(KArgs);
template __global__ void bwd_dq_ds_bf16_kernel<128>(KArgs);
template __global__ void bwd_dq_ds_bf16_kernel<192>(KArgs);
static_assert(DqDsCfg<128>::LDS_ELEMS * 2 * 2 <= 160 * 1024 && DqDsCfg<192>::LDS_ELEMS * 2 * 2 <= 160 * 1024,
              "two workgroups per CU");

hipError_t launch_bwd_dq_ds_bf16(const KArgs& a0, int dqk, int dv, hipStream_t stream) {
  (void)dv;  // dQ needs only K
  if (!a0.ds) return hipErrorInvalidValue;
  KArgs a = a0;
  a.n_tiles = (a.S + DqDsCfg<64>::BM - 1) / DqDsCfg<64>::BM;
  const dim3 grid((unsigned)(a.n_tiles * a.B * a.Hq));
  if (dqk == 64) hipLaunchKernelGGL((bwd_dq_ds_bf16_kernel<64>), grid, dim3(256), 0, stream, a);
  else if (dqk == 128) hipLaunchKernelGGL((bwd_dq_ds_bf16_kernel<128>), grid, dim3(256), 0, stream, a);
  else if (dqk == 192) hipLaunchKernelGGL((bwd_dq_ds_bf16_kernel<192>), grid, dim3(256), 0, stream, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace sdpa
