// Gradient of the attention bias, bf16 inputs, fp32 accumulation, gfx950 MFMA 32x32x16.
//
// With the bias read as an additive post-scale bias on the scores
// (s = scale q.k + bias; TE single-GPU page "Other attention knobs" passes a
// bias, PR #2225's backward returns grad_bias), its gradient for a bias matrix
// (b', h') is the sum, over the (batch, query head) pairs (b, h) that share it,
// of dS = P (dP - delta) on the pairs each of them sees (zero elsewhere):
//     P = exp(scale q.k + bias - LSE),  dP = dO V^T.
// Deterministic: a workgroup owns one block of the output and sums the
// sharing pairs in ascending order in registers; nothing is accumulated in
// memory.  Key tiles no sharing pair sees are written as zeros without
// reading the bias or recomputing anything.
//
// Work decomposition: 4 waves x 32 query rows (128 rows) of one bias matrix,
// over a range of key tiles of 64 keys.  Per key tile, for each sharing pair
// that sees any of it: K and V tiles of that pair's KV head are copied to LDS,
// the pair's Q and dO rows are loaded as register operands (as in the dQ
// kernel), S^T = K Q^T and dP^T = V dO^T are recomputed by MFMA (a lane owns
// a query row), and dS is added to the tile's fp32 accumulators.  delta and
// LSE * log2(e) come from the backward pre-pass in the workspace.  The tile is
// then written whole (zeros where no sharing pair sees it), so the output
// needs no clearing.
//
// On the stored-dS backward dS is already in the workspace and
// dbias_from_ds_kernel (end of this file) only sums it.
#include "dropout.h"
#include "launch.h"

namespace sdpa {

template <int DQK, int DV>
struct DbiasCfg {
  static constexpr int BM = 128, BN = 64, NT = 256;
  static constexpr int KCH = DQK / 8, VCH = DV / 8;
  static constexpr int KT = BN * DQK, VT = BN * DV;
  static constexpr int LDS_ELEMS = KT + VT;
};

template <int DQK, int DV, bool DROP>
__global__ __launch_bounds__(256, 2) void bwd_dbias_bf16_kernel(KArgs a) {
  using C = DbiasCfg<DQK, DV>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_ELEMS];
  uint16_t* Ks = lds;
  uint16_t* Vs = lds + C::KT;

  const int tid = threadIdx.x, w = wave_id(tid), lane = tid & 63, hf = lane >> 5, l32 = lane & 31;
  // Workgroup id -> (bias matrix, query tile, key-tile chunk).
  const int n_qt = a.n_tiles, n_kc = a.n_chunks;
  const int kc = blockIdx.x % n_kc;
  const int qt = (blockIdx.x / n_kc) % n_qt;
  const int mat = blockIdx.x / (n_kc * n_qt);
  const int bb = mat / a.bias_h, hh = mat % a.bias_h;  // the bias matrix (b', h')
  const int n_kt = (a.S + C::BN - 1) / C::BN;
  const int per_chunk = (n_kt + n_kc - 1) / n_kc;
  const int kt_lo = kc * per_chunk, kt_hi = kt_lo + per_chunk < n_kt ? kt_lo + per_chunk : n_kt;
  // Sharing pairs: all batches when bias_b == 1, all query heads when bias_h == 1.
  const int nb = a.bias_b == 1 ? a.B : 1, nh = a.bias_h == 1 ? a.Hq : 1;

  const int i0 = qt * C::BM, qw0 = i0 + w * 32, qi = qw0 + l32;
  const DropGen dg = drop_gen(a);
  const TileCopy<C::BN, C::KCH, C::NT> kcopy(tid, (uint32_t)(a.Hkv * DQK * 2));
  const TileCopy<C::BN, C::VCH, C::NT> vcopy(tid, (uint32_t)(a.Hkv * DV * 2));
  const RowReads<C::KCH> krd(lane);
  const RowReads<C::VCH> vrd(lane);
  RowBias<C::BN / 32> bias;
  bias.init(a, bb, hh, qi, hf);  // (b', h') is the matrix of every sharing pair
  const float c = a.scale_log2;
  const size_t qstride = (size_t)a.Hq * DQK, ostride = (size_t)a.Hq * DV;

  for (int kt = kt_lo; kt < kt_hi; ++kt) {
    const int j0 = kt * C::BN;
    bool seen = false;  // does any sharing pair see a (row, key) of the tile?
    for (int pb = 0; pb < nb && !seen; ++pb) {
      const MaskSpec m = make_mask(seq_len(a, a.bias_b == 1 ? pb : bb), a.S, a.causal, a.wl, a.wr);
      seen = tile_class(m, i0, C::BM, j0, C::BN) != TILE_SKIP;
    }
    if (!seen) {
      // The gradient is zero on the whole tile: 16-byte stores of zeros, eight
      // threads per row (S is a multiple of 8 and rows are 16-byte aligned, so
      // a chunk that starts below S lies wholly below it).
      uint16_t* out = static_cast<uint16_t*>(a.d_bias) + ((size_t)bb * a.bias_h + hh) * a.S * a.S;
#pragma unroll
      for (int r = 0; r < C::BM * C::BN / 8 / C::NT; ++r) {
        const int c = tid + r * C::NT, row = i0 + (c >> 3), key = j0 + (c & 7) * 8;
        if (row < a.S && key < a.S) *reinterpret_cast<u32x4*>(out + (size_t)row * a.S + key) = u32x4{0, 0, 0, 0};
      }
      continue;
    }
    f32x16 acc[C::BN / 32];
#pragma unroll
    for (int kb = 0; kb < C::BN / 32; ++kb) acc[kb] = f32x16{};
    bias.load(j0);
    for (int pb = 0; pb < nb; ++pb) {
      const int b = a.bias_b == 1 ? pb : bb;
      const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
      if (tile_class(m, i0, C::BM, j0, C::BN) == TILE_SKIP) continue;  // no row of the block sees it
      const size_t row0 = seq_row0(a, b);
      int klo, khi;
      row_key_bounds(m, qi, klo, khi);
      for (int ph = 0; ph < nh; ++ph) {
        const int h = a.bias_h == 1 ? ph : hh;
        const int g = h / a.G, bh = b * a.Hq + h;
        // K / V tiles of the pair's KV head; the previous pair's reads are
        // done (barrier at the end of the pair).
        kcopy.issue(static_cast<const uint16_t*>(a.k) + (row0 * a.Hkv + g) * DQK, (uint32_t)(a.Hkv * DQK * 2), j0,
                    m.L, Ks);
        vcopy.issue(static_cast<const uint16_t*>(a.v) + (row0 * a.Hkv + g) * DV, (uint32_t)(a.Hkv * DV * 2), j0, m.L,
                    Vs);
        // Q and dO rows of the pair (rows past the valid length read zeros),
        // and the rows' LSE * log2(e) and delta.
        bf16x8 qreg[DQK / 16], oreg[DV / 16];
        const __amdgpu_buffer_rsrc_t qres =
            buf_rsrc(static_cast<const uint16_t*>(a.q) + (row0 * a.Hq + h) * DQK, (uint32_t)(m.L * qstride * 2));
        const __amdgpu_buffer_rsrc_t ores =
            buf_rsrc(static_cast<const uint16_t*>(a.d_o) + (row0 * a.Hq + h) * DV, (uint32_t)(m.L * ostride * 2));
#pragma unroll
        for (int ks = 0; ks < DQK / 16; ++ks)
          qreg[ks] = as_bf16x8(buf_load16(qres, (uint32_t)(qi * qstride + ks * 16 + hf * 8) * 2));
#pragma unroll
        for (int ks = 0; ks < DV / 16; ++ks)
          oreg[ks] = as_bf16x8(buf_load16(ores, (uint32_t)(qi * ostride + ks * 16 + hf * 8) * 2));
        const size_t row = ((size_t)b * a.Hq + h) * a.S + (qi < a.S ? qi : a.S - 1);
        const float lse2 = qi < m.L ? a.lse2[row] : 0.0f;
        const float dl = qi < m.L ? a.delta[row] : 0.0f;
        uint32_t rnd[C::BN / 32][4];
        if constexpr (DROP) {
#pragma unroll
          for (int kb = 0; kb < C::BN / 32; ++kb) drop_rows_quad(dg, bh, qi, j0 + hf * 4 + kb * 32, rnd[kb]);
        }
        lds_dma_wait();
        __syncthreads();
        f32x16 st[C::BN / 32], dpt[C::BN / 32];
#pragma unroll
        for (int kb = 0; kb < C::BN / 32; ++kb) {
          st[kb] = f32x16{};
          dpt[kb] = f32x16{};
        }
#pragma unroll
        for (int ks = 0; ks < DQK / 16; ++ks)
#pragma unroll
          for (int kb = 0; kb < C::BN / 32; ++kb)
            st[kb] = mfma32(as_bf16x8(krd.read(Ks, kb * 32, ks)), qreg[ks], st[kb]);
#pragma unroll
        for (int ks = 0; ks < DV / 16; ++ks)
#pragma unroll
          for (int kb = 0; kb < C::BN / 32; ++kb)
            dpt[kb] = mfma32(as_bf16x8(vrd.read(Vs, kb * 32, ks)), oreg[ks], dpt[kb]);
        bias.add(st, a.inv_scale);
        // Element i of block kb: key j0 + kb*32 + acc_row(i, hf), query qi.
        const int lo_r = klo - (j0 + hf * 4), hi_r = khi - (j0 + hf * 4);
#pragma unroll
        for (int kb = 0; kb < C::BN / 32; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int off = kb * 32 + (i >> 2) * 8 + (i & 3);
            float pv = fast_exp2(fmaf(st[kb][i], c, -lse2));
            pv = (off >= lo_r && off <= hi_r) ? pv : 0.0f;
            float dpz = dpt[kb][i];
            if constexpr (DROP) dpz = drop_keep(rnd[kb][i >> 2], i & 3, dg.t) ? dpz * dg.scale : 0.0f;
            acc[kb][i] += pv * (dpz - dl);
          }
        __syncthreads();  // every wave is done with this pair's K / V tiles
      }
    }
    // Write the tile: rows below S, keys below S (four consecutive keys per
    // group of accumulator elements).
    if (qi < a.S) {
      uint16_t* out = static_cast<uint16_t*>(a.d_bias) + (((size_t)bb * a.bias_h + hh) * a.S + qi) * a.S;
#pragma unroll
      for (int kb = 0; kb < C::BN / 32; ++kb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int j = j0 + kb * 32 + gq * 8 + hf * 4;
          const float v[4] = {acc[kb][4 * gq], acc[kb][4 * gq + 1], acc[kb][4 * gq + 2], acc[kb][4 * gq + 3]};
          if (j + 3 < a.S) {
            *reinterpret_cast<u32x2*>(out + j) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (j + e < a.S) out[j + e] = (uint16_t)(pack_bf16(v[e], 0.0f) & 0xffffu);
          }
        }
    }
  }
}

template __global__ void bwd_dbias_bf16_kernel<64, 64, false>(KArgs);
template __global__ void bwd_dbias_bf16_kernel<128, 128, false>(KArgs);
template __global__ void bwd_dbias_bf16_kernel<64, 64, true>(KArgs);
template __global__ void bwd_dbias_bf16_kernel<128, 128, true>(KArgs);

// Key-tile chunks per (bias matrix, query tile) so that the grid holds about
// 2048 workgroups (broadcast biases have few matrices, each summing many pairs).
int dbias_key_chunks(int n_mats, int n_qt, int n_kt) {
  const long long base = (long long)n_mats * n_qt;
  long long want = (2048 + base - 1) / base;
  if (want > n_kt) want = n_kt;
  return want < 1 ? 1 : (int)want;
}

template <int DQK, int DV>
static hipError_t launch_dbias_cfg(KArgs a, hipStream_t stream) {
  using C = DbiasCfg<DQK, DV>;
  a.n_tiles = (a.S + C::BM - 1) / C::BM;
  const int n_kt = (a.S + C::BN - 1) / C::BN;
  a.n_chunks = dbias_key_chunks(a.bias_b * a.bias_h, a.n_tiles, n_kt);
  const dim3 grid((unsigned)(a.bias_b * a.bias_h * a.n_tiles * a.n_chunks));
  if (a.drop_t > 0) hipLaunchKernelGGL((bwd_dbias_bf16_kernel<DQK, DV, true>), grid, dim3(C::NT), 0, stream, a);
  else hipLaunchKernelGGL((bwd_dbias_bf16_kernel<DQK, DV, false>), grid, dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bwd_dbias_bf16(const KArgs& a, int dqk, int dv, hipStream_t stream) {
  if (dqk == 64 && dv == 64) return launch_dbias_cfg<64, 64>(a, stream);
  if (dqk == 128 && dv == 128) return launch_dbias_cfg<128, 128>(a, stream);
  return hipErrorInvalidValue;
}

// ---- dBias from the stored dS ------------------------------------------------
//
// On the stored-dS backward the dK/dV kernel has written every visible 32-row
// x 32-key block of dS (times ds_stored_sign, in its register order: lane l
// of key group w holds key w*32 + l%32 and rows acc_row(i, l/32), i = 0..15,
// 32 bytes at w*2048 + l*32 of the 8 KiB block of 32 rows x 128 keys).  dBias of a bias
// matrix is then the sum of those blocks over the sharing (batch, query head)
// pairs, in ascending pair order, with no recomputation.  A workgroup owns
// kDbRowBlocks blocks of 32 rows x 128 keys of one bias matrix, one after the
// other: each thread adds up one key's 16 rows over the pairs whose block
// exists (the tests the dK/dV kernel stores by: the key tile's slab range at
// the batch's length, and tile_class of the 32 x 32 block), the block is
// transposed through LDS and written as whole 16-byte row pieces, zeros where
// no pair sees it.
constexpr int kDbRowBlocks = 4;

// First block of key tile kt's slab (ds_slab's `first`), the tiles before it
// dealt over a wave's lanes and summed: these workgroups are small, and the
// one-lane loop of ds_slab would cost more than their memory traffic.
__device__ __forceinline__ int ds_slab_first_lanes(const KArgs& a, int kt, int lane) {
  const MaskSpec mf = make_mask(a.S, a.S, a.causal, a.wl, a.wr);
  int n = 0;
  for (int t = lane; t < kt; t += 64) n += ds_tile_blocks(mf, t);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o);
  return __builtin_amdgcn_readfirstlane(n);
}

__global__ __launch_bounds__(256) void dbias_from_ds_kernel(KArgs a) {
  __shared__ float tile[32][128 + 4];
  const int tid = threadIdx.x, w = wave_id(tid), lane = tid & 63, l32 = lane & 31, hf = lane >> 5;
  const int n_kt = (a.S + 127) / 128, n_rc = (a.S + 32 * kDbRowBlocks - 1) / (32 * kDbRowBlocks);
  const int kt = blockIdx.x % n_kt;
  const int rc = (blockIdx.x / n_kt) % n_rc;
  const int mat = blockIdx.x / (n_kt * n_rc);
  const int bb = mat / a.bias_h, hh = mat % a.bias_h;
  const int nb = a.bias_b == 1 ? a.B : 1, nh = a.bias_h == 1 ? a.Hq : 1;
  const int k0 = kt * 128 + w * 32;  // this wave's key group
  const int first = ds_slab_first_lanes(a, kt, lane);
  const int count = ds_tile_blocks(make_mask(a.S, a.S, a.causal, a.wl, a.wr), kt);
  uint16_t* out = static_cast<uint16_t*>(a.d_bias) + ((size_t)bb * a.bias_h + hh) * a.S * a.S;
  const float sgn = ds_stored_sign(a);
  for (int j = 0; j < kDbRowBlocks; ++j) {
    const int r0 = (rc * kDbRowBlocks + j) * 32;
    if (r0 >= a.S) break;
    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    for (int bi = 0; bi < nb; ++bi) {
      const int b = a.bias_b == 1 ? bi : bb;
      const MaskSpec m = make_mask(seq_len(a, b), a.S, a.causal, a.wl, a.wr);
      int qlo, qhi;
      if (!query_range(m, kt * 128, kt * 128 + 127, qlo, qhi)) continue;
      int nblk = 2 * (qhi / 64 - qlo / 64 + 1);
      nblk = nblk < count ? nblk : count;
      const int r = (r0 - (qlo / 64) * 64) >> 5;
      if (r < 0 || r >= nblk || tile_class(m, r0, 32, k0, 32) == TILE_SKIP) continue;
#pragma unroll 4
      for (int hi = 0; hi < nh; ++hi) {
        const int h = a.bias_h == 1 ? hi : hh;
        const uint16_t* blk =
            a.ds + ((size_t)(b * a.Hq + h) * a.ds_head_blocks + first + r) * 4096 + w * 1024 + lane * 16;
        // read once: non-temporal loads
        const u32x4 v0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(blk));
        const u32x4 v1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(blk + 8));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += bf16_lo(v0[e]);
          acc[2 * e + 1] += bf16_hi(v0[e]);
          acc[8 + 2 * e] += bf16_lo(v1[e]);
          acc[8 + 2 * e + 1] += bf16_hi(v1[e]);
        }
      }
    }
    if (j > 0) __syncthreads();  // the previous block's rows are read out
#pragma unroll
    for (int i = 0; i < 16; ++i) tile[acc_row(i, hf)][w * 32 + l32] = sgn * acc[i];
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int c = tid + 256 * k, row = c >> 4, kc = (c & 15) * 8;
      const int gr = r0 + row, gk = kt * 128 + kc;
      if (gr < a.S && gk < a.S) {
        const float* t = &tile[row][kc];
        *reinterpret_cast<u32x4*>(out + (size_t)gr * a.S + gk) =
            u32x4{pack_bf16(t[0], t[1]), pack_bf16(t[2], t[3]), pack_bf16(t[4], t[5]), pack_bf16(t[6], t[7])};
      }
    }
  }
}

hipError_t launch_dbias_from_ds(const KArgs& a, hipStream_t stream) {
  if (!a.ds || !a.d_bias) return hipErrorInvalidValue;
  const long long n = (long long)a.bias_b * a.bias_h * ((a.S + 127) / 128) *
                      ((a.S + 32 * kDbRowBlocks - 1) / (32 * kDbRowBlocks));
  if (n > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dbias_from_ds_kernel, dim3((unsigned)n), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sdpa
