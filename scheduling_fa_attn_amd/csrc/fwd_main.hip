// Forward HIP kernel of softmax attention for gfx950 (MI355X): O and the natural-log
// LSE of every query row, the inputs the backward pass recomputes its probabilities from.
//
// Math ("Writing an Attention Kernel", Step 1 for the definition, Step 2 for the tiled
// online softmax; DASH paper section 2.1 for the role of the LSE): per (b, h) and query
// row q, with scores S[k] = s q.K[k] (masked keys -inf),
//   LSE[q] = log sum_k exp(S[k]),   O[q] = sum_k exp(S[k] - LSE[q]) V[k].
// Key tiles are visited in ascending order with a running maximum m and a running sum l
// per row: for each tile, m' = max(m, max_tile S), O <- O exp(m - m') + P V and
// l <- l exp(m - m') + sum P with P = exp(S - m'); at the end O /= l, LSE = m + log l.
// Everything is computed in base 2 with log2(e) folded into the scale.
//
// CDNA4 mapping
// - One workgroup of 4 waves per (b, h, 128-row Q tile); wave w owns query rows
//   q0 + 32 w .. + 31. Two workgroups fit on a CU at d = 128 (68 KiB of LDS, at most 256
//   registers per lane) and four at d = 64, so every SIMD interleaves several waves.
// - The wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16: A = 32 key rows from
//   LDS, B = the wave's query rows, held in registers for the whole kernel. In the S^T
//   accumulator a lane holds one query row (column lane % 32) and 16 keys, so the row
//   maximum and sum need only the lane's own values and the other half-wave's.
// - O^T = V^T P^T accumulates in the same orientation (a lane holds one query row, all
//   of d over its 4 d blocks), so the rescale by exp(m - m') is the lane's own factor.
//   A = V^T from transpose reads of the V tile (ds_read_b64_tr_b16), B = P^T straight from
//   the S^T accumulator as bf16 pairs: element r of a 32-key block is key 8 (r / 4) +
//   4 hi + r % 4, so the k-step over keys 16 u .. 16 u + 15 (u = 0, 1 within a block)
//   takes elements 8 u .. 8 u + 7, and the A operand reads key rows in the same order.
// - Key tiles of 64 rows; K and V tiles are double-buffered in LDS and copied global ->
//   LDS one tile ahead (global_load_lds, as the backward's tiles).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace dash {

template <int D>
struct FwdCfg {
  static constexpr int NW = 4;                     // waves
  static constexpr int BQ = 32 * NW;               // query rows per workgroup
  static constexpr int BK = 64;                    // key rows per tile
  static constexpr int ST = TileGeom<D>::STRIDE;   // LDS row stride
  static constexpr int KT = BK * ST;               // bytes of one K (or V) tile
  static constexpr int DK = D / 16;                // k-steps over d
  static constexpr int DB = D / 32;                // 32-column blocks of d
  static constexpr int BYTES = 4 * KT;             // K[2], V[2]
};

// Waves per SIMD: 2 at d = 128 (176 VGPRs, 68 KiB of LDS per workgroup); 4 at d = 64,
// where a workgroup needs at most 128 VGPRs per lane and 36 KiB of LDS (measured 11 %
// faster on causal d = 64 N = 4096 than 2).
template <int D>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(D == 64 ? 4 : 2, D == 64 ? 4 : 2)))
fwd_kernel(FwdParams p) {
  using C = FwdCfg<D>;
  constexpr int NW = C::NW, BQ = C::BQ, BK = C::BK, ST = C::ST, KT = C::KT, DK = C::DK, DB = C::DB;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int L16 = lane & 15;
  const int N = p.N;

  // Workgroup -> (Q tile, b * H + h); with the causal mask the longest Q tiles (the last
  // ones) are dispatched first.
  const int heads = p.B * p.H;
  const int qt = p.n_qt - 1 - static_cast<int>(blockIdx.x / heads);
  const int bh = static_cast<int>(blockIdx.x % heads);
  const int b = bh / p.H, h = bh % p.H;
  const int64_t bg = static_cast<int64_t>(b) * p.Hkv + h / (p.H / p.Hkv);
  const int q0 = qt * BQ;
  const bf16* kg = p.k + bg * N * D;
  const bf16* vg = p.v + bg * N * D;
  const int n_kv_all = (N + BK - 1) / BK;
  const int n_kv_causal = (q0 + BQ + BK - 1) / BK;
  const int n_kv = p.causal && n_kv_causal < n_kv_all ? n_kv_causal : n_kv_all;

  TileCopy<D, BK, NW> copy;
  copy.init(w, lane);
  copy.issue(smem, kg, 0, N, w);
  copy.issue(smem + 2 * KT, vg, 0, N, w);

  // This lane's query row (rows past N read row N - 1 and are never stored); the B
  // operand of k-step ks holds its d columns 16 ks + 8 hi .. + 7.
  const int qrow = q0 + 32 * w + l32;
  const int qread = qrow < N ? qrow : N - 1;
  bf16x8 qreg[DK];
#pragma unroll
  for (int ks = 0; ks < DK; ++ks)
    qreg[ks] = *reinterpret_cast<const bf16x8*>(p.q + (static_cast<int64_t>(bh) * N + qread) * D + 16 * ks + 8 * hi);

  floatx16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = floatx16{};
  float m = -__builtin_inff();  // running maximum of s log2(e) S over this lane's row
  float l = 0.f;                // running sum of this half-wave's probabilities
  const float c = p.scale_log2;

  // Transpose-read addresses of the V^T operand: lane group (lane / 16) reads column
  // block n0 = 32 db + 16 ((lane / 16) % 2); its lane supplies row (L16 / 4) of the 4 key
  // rows and columns n0 + 4 (L16 % 4) .. + 3.
  const int vt_lane = (L16 >> 2) * ST + 2 * (16 * ((lane >> 4) & 1) + 4 * (L16 & 3));

  for (int t = 0; t < n_kv; ++t) {
    const int buf = t & 1;
    // Tile t has landed (this wave's copies, then everyone's); every wave is done with
    // tile t - 1, whose buffers the copies of tile t + 1 overwrite.
    wait_mem_done();
    __syncthreads();
    if (t + 1 < n_kv) {
      copy.issue(smem + (buf ^ 1) * KT, kg, (t + 1) * BK, N, w);
      copy.issue(smem + (2 + (buf ^ 1)) * KT, vg, (t + 1) * BK, N, w);
    }
    const LDS_AS char* sK = smem + buf * KT;
    const LDS_AS char* sV = smem + (2 + buf) * KT;
    const int kv0 = t * BK;

    // S^T of key blocks kb = 0, 1 (keys kv0 + 32 kb .. + 31).
    floatx16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = floatx16{};
#pragma unroll
      for (int ks = 0; ks < DK; ++ks)
        s[kb] = mfma32(lds_ld16(sK, (32 * kb + l32) * ST + 32 * ks + 16 * hi), qreg[ks], s[kb]);
    }
    // Masks: keys past N; with the causal mask, keys after the query row.
    const bool ragged = kv0 + BK > N;
    const bool diag = p.causal && kv0 + BK - 1 > q0;
    if (ragged || diag) {
      const int lim = p.causal && qrow < N - 1 ? qrow : N - 1;  // last visible key
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kv = kv0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (kv > lim) s[kb][r] = -__builtin_inff();
        }
    }
    // Online softmax of this lane's row.
    float mt = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = __builtin_fmaxf(mt, s[kb][r]);
    mt = __builtin_fmaxf(mt, __shfl_xor(mt, 32));
    const float m_new = __builtin_fmaxf(m, mt * c);
    // A row whose keys are all masked so far keeps m = -inf; exp2(-inf - 0) = 0 keeps it empty.
    const float m_use = m_new == -__builtin_inff() ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    m = m_new;
    u32x4 pk[2][2];
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -m_use));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], c, -m_use));
        lsum += p0 + p1;
        pk[kb][r >> 3][(r & 7) >> 1] = pack_bf16(p0, p1);
      }
    l = l * alpha + lsum;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    // O^T += V^T P^T over the tile's 64 keys (k-steps kk = 2 kb + u).
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int kb = kk >> 1, u = kk & 1;
      const int row0 = 32 * kb + 16 * u + 4 * hi;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int off = vt_lane + row0 * ST + 64 * db;
        const bf16x8 a = join(lds_tr(sV, off), lds_tr(sV, off + 8 * ST));
        o[db] = mfma32(a, as_bf16x8(pk[kb][u]), o[db]);
      }
    }
  }

  // Epilogue: O = O^T / l, LSE = (m + log2 l) ln 2 of this lane's row.
  const float l_tot = l + __shfl_xor(l, 32);
  const float inv = 1.f / l_tot;
  if (qrow < N) {
    bf16* orow = p.o + (static_cast<int64_t>(bh) * N + qrow) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        // Elements 4 g4 .. 4 g4 + 3: d = 32 db + 8 g4 + 4 hi + 0 .. 3.
        u32x2 x;
        x[0] = pack_bf16(o[db][4 * g4] * inv, o[db][4 * g4 + 1] * inv);
        x[1] = pack_bf16(o[db][4 * g4 + 2] * inv, o[db][4 * g4 + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * g4 + 4 * hi) = x;
      }
    if (hi == 0) p.lse[static_cast<int64_t>(bh) * N + qrow] = (m + __builtin_log2f(l_tot)) * 0.6931471805599453f;
  }
}

template <int D>
static hipError_t launch_fwd_t(const FwdParams& prm, hipStream_t stream) {
  using C = FwdCfg<D>;
  const int64_t grid = static_cast<int64_t>(prm.B) * prm.H * prm.n_qt;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fwd_kernel<D>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, C::BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fwd_kernel<D>, dim3(static_cast<unsigned>(grid)), dim3(C::NW * 64), C::BYTES, stream, prm);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams& prm, int d, hipStream_t stream) {
  if (d == 64) return launch_fwd_t<64>(prm, stream);
  if (d == 128) return launch_fwd_t<128>(prm, stream);
  return hipErrorInvalidValue;
}

}  // namespace dash
