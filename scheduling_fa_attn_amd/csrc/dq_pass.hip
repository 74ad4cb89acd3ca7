// dQ pass of the two-pass deterministic backward for gfx950 (MI355X).
//
// The DASH paper (section 5, related work) contrasts its ordered cross-CU reduction with
// designs that compute dQ in a pass of its own: each query tile walks all key tiles and
// keeps its dQ in registers, so no partial sum ever leaves the compute unit and the
// result is deterministic with no ordering protocol, at the price of recomputing S and dP
// (three of the backward's five contractions run twice in total). This kernel is that
// pass; dK and dV come from the main kernel with its dQ work switched off.
//
// Math (DASH paper section 2.1; "Writing an Attention Kernel", section "In the real world"),
// per (b, h) and query row q, over the keys k it sees:
//   P[k] = exp(s q.K[k] - LSE[q]),  dP[k] = dO[q].V[k],  dS[k] = P[k] (dP[k] - D[q]),
//   dQ[q] = s sum_k dS[k] K[k],  with D = rowsum(dO * O) from the preprocess.
//
// CDNA4 mapping (the forward kernel's): one workgroup of 4 waves per (b, h, 128-row Q
// tile), two workgroups per CU. Each wave computes S^T = K Q^T and dP^T = V dO^T
// (v_mfma_f32_32x32x16_bf16; A = 32 key rows of the K or V tile from LDS, B = the wave's
// 32 query rows of Q or dO, held in registers), so that a lane holds one query row and
// its -LSE*log2(e) and -D are that lane's scalars; then dQ^T += K^T dS^T with A = K^T from
// transpose reads of the K tile and B = dS^T straight from the registers as bf16 pairs.
// Key tiles of 64 rows, K and V double-buffered in LDS and copied one tile ahead.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace dash {

template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
dq_pass_kernel(DqParams p) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *p.status_out = *p.err_in;
  constexpr int NW = 4, BQ = 32 * NW, BK = 64, ST = TileGeom<D>::STRIDE, KT = BK * ST, DK = D / 16, DB = D / 32;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int L16 = lane & 15;
  const int N = p.N;

  const int heads = p.B * p.H;
  const int qt = p.n_qt - 1 - static_cast<int>(blockIdx.x / heads);
  const int bh = static_cast<int>(blockIdx.x % heads);
  const int b = bh / p.H, h = bh % p.H;
  const int64_t bg = static_cast<int64_t>(b) * p.Hkv + h / (p.H / p.Hkv);
  const int q0 = qt * BQ;
  // Rows of this batch: N, or its length for variable-length batches (N stays the row
  // stride; rows past the length are padding, never read as data or written).
  const int nb = p.seqlens ? p.seqlens[b] : N;
  if (q0 >= nb) return;  // a Q tile wholly past the batch's length (uniform: no barrier missed)
  const bf16* kg = p.k + bg * N * D;
  const bf16* vg = p.v + bg * N * D;
  const int n_kv_all = (nb + BK - 1) / BK;
  const int n_kv_causal = (q0 + BQ + BK - 1) / BK;
  const int n_kv = p.causal && n_kv_causal < n_kv_all ? n_kv_causal : n_kv_all;

  TileCopy<D, BK, NW> copy;
  copy.init(w, lane);
  copy.issue(smem, kg, 0, nb, w);
  copy.issue(smem + 2 * KT, vg, 0, nb, w);

  // This lane's query row (rows past the length read its last row and are never stored).
  const int qrow = q0 + 32 * w + l32;
  const int qread = qrow < nb ? qrow : nb - 1;
  bf16x8 qreg[DK], doreg[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks) {
    const int64_t off = (static_cast<int64_t>(bh) * N + qread) * D + 16 * ks + 8 * hi;
    qreg[ks] = *reinterpret_cast<const bf16x8*>(p.q + off);
    doreg[ks] = *reinterpret_cast<const bf16x8*>(p.dO + off);
  }
  // Row terms of this lane's row (row arrays are padded to the tile: -LSE*log2(e) is
  // -inf and -D is 0 past the length).
  const float nl = p.nlse2[static_cast<int64_t>(bh) * p.row_stride + qread];
  const float nd = p.neg_delta[static_cast<int64_t>(bh) * p.row_stride + qread];
  const float c = p.scale_log2;

  floatx16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = floatx16{};
  // Transpose-read addresses of the K^T operand (as the forward's V^T).
  const int kt_lane = (L16 >> 2) * ST + 2 * (16 * ((lane >> 4) & 1) + 4 * (L16 & 3));

  for (int t = 0; t < n_kv; ++t) {
    const int buf = t & 1;
    wait_mem_done();
    __syncthreads();
    if (t + 1 < n_kv) {
      copy.issue(smem + (buf ^ 1) * KT, kg, (t + 1) * BK, nb, w);
      copy.issue(smem + (2 + (buf ^ 1)) * KT, vg, (t + 1) * BK, nb, w);
    }
    const LDS_AS char* sK = smem + buf * KT;
    const LDS_AS char* sV = smem + (2 + buf) * KT;
    const int kv0 = t * BK;
    floatx16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = floatx16{};
      dp[kb] = floatx16{};
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        const int off = (32 * kb + l32) * ST + 32 * ks + 16 * hi;
        s[kb] = mfma32(lds_ld16(sK, off), qreg[ks], s[kb]);
        dp[kb] = mfma32(lds_ld16(sV, off), doreg[ks], dp[kb]);
      }
    }
    const bool ragged = kv0 + BK > nb;
    const bool diag = p.causal && kv0 + BK - 1 > q0;
    if (ragged || diag) {
      const int lim = p.causal && qrow < nb - 1 ? qrow : nb - 1;  // last visible key
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kv = kv0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (kv > lim) s[kb][r] = -__builtin_inff();
        }
    }
    // dS^T as bf16 pairs: element r of key block kb is key 8 (r / 4) + 4 hi + r % 4.
    u32x4 pk[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, nl));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], c, nl));
        pk[kb][r >> 3][(r & 7) >> 1] = pack_bf16(p0 * (dp[kb][r] + nd), p1 * (dp[kb][r + 1] + nd));
      }
    // dQ^T += K^T dS^T over the tile's 64 keys (k-steps kk = 2 kb + u).
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kb = kk >> 1, u = kk & 1;
      const int row0 = 32 * kb + 16 * u + 4 * hi;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int off = kt_lane + row0 * ST + 64 * db;
        const bf16x8 a = join(lds_tr(sK, off), lds_tr(sK, off + 8 * ST));
        acc[db] = mfma32(a, as_bf16x8(pk[kb][u]), acc[db]);
      }
    }
  }

  // dQ = s dQ^T: elements 4 g4 .. 4 g4 + 3 of block db are d = 32 db + 8 g4 + 4 hi + 0 .. 3.
  if (qrow < nb) {
    bf16* row = p.dq + (static_cast<int64_t>(bh) * N + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 x;
        x[0] = pack_bf16(acc[db][4 * g4] * p.scale, acc[db][4 * g4 + 1] * p.scale);
        x[1] = pack_bf16(acc[db][4 * g4 + 2] * p.scale, acc[db][4 * g4 + 3] * p.scale);
        *reinterpret_cast<u32x2*>(row + 32 * db + 8 * g4 + 4 * hi) = x;
      }
  }
}

template <int D>
static hipError_t launch_dq_pass_t(const DqParams& prm, hipStream_t stream) {
  constexpr int bytes = 4 * 64 * TileGeom<D>::STRIDE;
  const int64_t grid = static_cast<int64_t>(prm.B) * prm.H * prm.n_qt;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(dq_pass_kernel<D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dq_pass_kernel<D>, dim3(static_cast<unsigned>(grid)), dim3(256), bytes, stream, prm);
  return hipGetLastError();
}

hipError_t launch_dq_pass(const DqParams& prm, int d, hipStream_t stream) {
  if (d == 64) return launch_dq_pass_t<64>(prm, stream);
  if (d == 128) return launch_dq_pass_t<128>(prm, stream);
  return hipErrorInvalidValue;
}

}  // namespace dash
