// Auxiliary HIP kernels of the attention backward for gfx950: the preprocess
// (D = rowsum(dO * O), -LSE*log2(e), clearing), the dQ casts of the ordered and the
// atomic variant and the XCD topology probe.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

namespace dash {

// ---------------------------------------------------------------------------------
// Preprocess: -D[row] = -sum_e dO[row, e] * O[row, e] in fp32 with a fixed reduction
// tree and nl[row] = -LSE[row] * log2(e), stored with the head's rows padded to the
// tile (padding: -D = 0, nl = -inf); clears the ordering semaphores, the XCD slot
// counters and the call's error word; for the atomic variant also clears the fp32 dQ
// accumulator.
// (-D is stored negated because the main kernel starts its dP = dO V^T accumulation
// from it, which yields dP - D directly.)
// ---------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256) preprocess_kernel(PreParams p) {
  constexpr int LPR = D / 8;  // lanes per row, 8 elements (16 bytes) per lane
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int64_t rows = p.rows;
  for (int64_t base = tid; base < rows * LPR; base += nthreads) {
    const int64_t row = base / LPR;
    const int part = static_cast<int>(base % LPR);
    const bf16x8 ov = *reinterpret_cast<const bf16x8*>(p.o + row * D + part * 8);
    const bf16x8 dv = *reinterpret_cast<const bf16x8*>(p.dO + row * D + part * 8);
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(static_cast<float>(ov[e]), static_cast<float>(dv[e]), acc);
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) acc += __shfl_xor(acc, off, LPR);
    if (part == 0) {
      const int64_t bh = row / p.N;
      const int r = static_cast<int>(row % p.N);
      const int64_t out = bh * p.row_stride + r;
      // Variable-length batches: rows past the batch's length are padding, like rows
      // past N (their inputs are never read as data).
      const bool valid = !p.seqlens || r < p.seqlens[bh / p.H];
      p.neg_delta[out] = valid ? -acc : 0.f;
      p.nlse2[out] = valid ? -p.lse[row] * 1.4426950408889634f : -__builtin_inff();
    }
  }
  // Rows past N (up to the tile boundary): P = exp2(S * c - inf) = 0 there, dS = 0.
  const int pad = p.row_stride - p.N;
  if (pad > 0) {
    const int64_t heads = p.rows / p.N;
    for (int64_t x = tid; x < heads * pad; x += nthreads) {
      const int64_t out = (x / pad) * p.row_stride + p.N + x % pad;
      p.neg_delta[out] = 0.f;
      p.nlse2[out] = -__builtin_inff();
    }
  }
  for (int64_t x = tid; x < p.sem_count; x += nthreads) p.sem[x] = 0;
  for (int64_t x = tid; x < p.ctr_count; x += nthreads) p.ctr[x] = 0;
  if (tid == 0) *p.err = 0;
  if (p.dqacc_zero) {
    floatx4* z = reinterpret_cast<floatx4*>(p.dqacc_zero);
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int64_t x = tid; x < p.zero_count / 4; x += nthreads) z[x] = zero;
  }
}

// The call's error word into the stream's status slot, for calls with no cast kernel
// (the two-waves kernel writes dQ itself in the ordered variant).
__global__ void __launch_bounds__(64) status_copy_kernel(StatusCopy sc) {
  if (threadIdx.x == 0) *sc.status_out = *sc.err_in;
}

hipError_t launch_status_copy(StatusCopy sc, hipStream_t stream) {
  hipLaunchKernelGGL(status_copy_kernel, dim3(1), dim3(64), 0, stream, sc);
  return hipGetLastError();
}

// dQ = bf16(s * dQacc), for the ordered variant of the one-wave kernel: the accumulator
// holds the final fp32 sums in the block layout described at kDqBlock. One workgroup per
// 32-row block row of one head reads its D / 32 blocks with 16-byte loads, rounds them,
// puts them in row order in LDS and writes rows < N in 16-byte chunks. (The two-waves
// kernel's last contributors write bf16 dQ themselves, transposed in registers.)
template <int D>
__global__ void __launch_bounds__(256) dq_cast_blocks_kernel(const float* __restrict__ acc, bf16* __restrict__ dq,
                                                             int N, int row_stride, float scale,
                                                             const int* __restrict__ seqlens, int H, StatusCopy sc) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *sc.status_out = *sc.err_in;
  constexpr int DB = D / 32;
  constexpr int LROW = D + 8;  // bf16 per LDS row (16-byte pad)
  __shared__ __attribute__((aligned(16))) bf16 tile[32 * LROW];
  const int rbs = row_stride / 32;  // block rows per head
  const int64_t g = blockIdx.x;     // (head, block row)
  const int64_t bh = g / rbs;
  const int qblk = static_cast<int>(g % rbs);
  const floatx4* src = reinterpret_cast<const floatx4*>(acc + g * DB * kDqBlock);
#pragma unroll
  for (int k = 0; k < DB; ++k) {
    // float4 x of the block row: block db = x / 256; floats 4 l + 256 i .. + 3 of block db
    // are elements 4 i .. 4 i + 3 of lane l: rows 16 (i / 2) + 2 (i % 2) + l / 32 + 4 e,
    // column 32 db + l % 32.
    const int x = threadIdx.x + 256 * k;
    const int db = x >> 8, i = (x >> 6) & 3, l = x & 63;
    const floatx4 v = src[x];
    const int row0 = 16 * (i >> 1) + 2 * (i & 1) + (l >> 5);
    const int col = 32 * db + (l & 31);
#pragma unroll
    for (int e = 0; e < 4; ++e) tile[(row0 + 4 * e) * LROW + col] = static_cast<bf16>(v[e] * scale);
  }
  __syncthreads();
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  // Rows < N (variable-length batches: < the batch's length) are written; rows past it
  // are left as they are.
  const int nb = seqlens ? seqlens[bh / H] : N;
  const int r_end = nb - 32 * qblk < 32 ? nb - 32 * qblk : 32;
#pragma unroll
  for (int k = 0; k < 32 * CPR / 256; ++k) {
    const int c = threadIdx.x + 256 * k;
    const int r = c / CPR, ch = c % CPR;
    if (r < r_end) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(&tile[r * LROW + 8 * ch]);
      *reinterpret_cast<u32x4*>(dq + (bh * N + 32 * qblk + r) * D + 8 * ch) = v;
    }
  }
}

// dQ of the per-tile partials variant (deterministic = 3; the deterministic alternative of
// the DASH paper, section 5: every KV tile's dQ contribution materialised, then reduced by a
// separate kernel): dQ = bf16(s * sum of the contributions of each 64-row step), added in
// fp32 in rank order from +0 (the slot layout is described at kDqBlock). One workgroup per
// 32-row block row of one head, as in dq_cast_blocks_kernel: each thread owns 4 floats of
// each of the block row's D / 32 blocks and walks the step's slots.
template <int D>
__global__ void __launch_bounds__(256) dq_consolidate_kernel(const float* __restrict__ parts, bf16* __restrict__ dq,
                                                             int N, int row_stride, int tile, int causal,
                                                             float scale, StatusCopy sc) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *sc.status_out = *sc.err_in;
  constexpr int DB = D / 32;
  constexpr int LROW = D + 8;
  constexpr int SLOT4 = 2 * DB * kDqBlock / 4;  // float4 per slot
  __shared__ __attribute__((aligned(16))) bf16 lds[32 * LROW];
  const int rbs = row_stride / 32;
  const int64_t g = blockIdx.x;
  const int64_t bh = g / rbs;
  const int qblk = static_cast<int>(g % rbs);
  const int q0 = (qblk / 2) * 64;  // the block row's 64-row step
  const int qb = qblk % 2;         // and its half of that step
  const int n = row_stride / tile;
  const int j = q0 / tile;
  const int cnt = causal ? j + 1 : n;
  const floatx4* slots = reinterpret_cast<const floatx4*>(parts) + partial_slot(bh, q0, 0, n, tile, causal) * SLOT4;
#pragma unroll
  for (int k = 0; k < DB; ++k) {
    const int x = threadIdx.x + 256 * k;
    const int db = x >> 8, i = (x >> 6) & 3, l = x & 63;
    const floatx4* src = slots + (qb * DB + db) * (kDqBlock / 4) + (x & 255);
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int r = 0; r < cnt; ++r) acc = acc + src[static_cast<int64_t>(r) * SLOT4];
    const int row0 = 16 * (i >> 1) + 2 * (i & 1) + (l >> 5);
    const int col = 32 * db + (l & 31);
#pragma unroll
    for (int e = 0; e < 4; ++e) lds[(row0 + 4 * e) * LROW + col] = static_cast<bf16>(acc[e] * scale);
  }
  __syncthreads();
  constexpr int CPR = D / 8;
  const int r_end = N - 32 * qblk < 32 ? N - 32 * qblk : 32;
#pragma unroll
  for (int k = 0; k < 32 * CPR / 256; ++k) {
    const int c = threadIdx.x + 256 * k;
    const int r = c / CPR, ch = c % CPR;
    if (r < r_end) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(&lds[r * LROW + 8 * ch]);
      *reinterpret_cast<u32x4*>(dq + (bh * N + 32 * qblk + r) * D + 8 * ch) = v;
    }
  }
}

// dQ = bf16(s * dQacc), for the atomic variant; the accumulator is row-major with
// row_stride rows per head, of which the first N are output.
__global__ void __launch_bounds__(256) dq_cast_kernel(const float* __restrict__ acc, bf16* __restrict__ dq,
                                                      int64_t quads, int N, int row_stride, int d, float scale,
                                                      const int* __restrict__ seqlens, int H, StatusCopy sc) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *sc.status_out = *sc.err_in;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const int qpr = d / 4;  // float4 per row
  for (int64_t x = tid; x < quads; x += nthreads) {
    const int64_t row_all = x / qpr;
    const int col = static_cast<int>(x % qpr) * 4;
    const int64_t bh = row_all / N;
    const int row = static_cast<int>(row_all % N);
    if (seqlens && row >= seqlens[bh / H]) continue;  // padding of a shorter batch: left as it is
    const floatx4 a = *reinterpret_cast<const floatx4*>(acc + (bh * row_stride + row) * d + col);
    bf16x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = static_cast<bf16>(a[e] * scale);
    *reinterpret_cast<bf16x4*>(dq + row_all * d + col) = r;
  }
}

// Records the XCD of every workgroup of a one-workgroup-per-CU grid.
__global__ void __launch_bounds__(64) topology_probe_kernel(int* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = static_cast<int>(xcc_id());
}

hipError_t launch_preprocess(const PreParams& prm, int d, int grid, hipStream_t stream) {
  if (d == 64) {
    hipLaunchKernelGGL(preprocess_kernel<64>, dim3(grid), dim3(256), 0, stream, prm);
  } else if (d == 128) {
    hipLaunchKernelGGL(preprocess_kernel<128>, dim3(grid), dim3(256), 0, stream, prm);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dq_cast(const float* acc, void* dq, int64_t heads, int N, int row_stride, int d, float scale,
                          StatusCopy sc, hipStream_t stream, const int* seqlens, int H) {
  const int64_t quads = heads * N * (d / 4);
  int64_t grid = (quads + 255) / 256;
  grid = grid < 1 ? 1 : (grid > 8192 ? 8192 : grid);
  hipLaunchKernelGGL(dq_cast_kernel, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, acc,
                     reinterpret_cast<bf16*>(dq), quads, N, row_stride, d, scale, seqlens, H, sc);
  return hipGetLastError();
}

hipError_t launch_dq_consolidate(const float* parts, void* dq, int64_t heads, int N, int row_stride, int tile, int d,
                                 int causal, float scale, StatusCopy sc, hipStream_t stream) {
  const int64_t grid = heads * (row_stride / 32);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (d == 64) {
    hipLaunchKernelGGL(dq_consolidate_kernel<64>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, parts,
                       reinterpret_cast<bf16*>(dq), N, row_stride, tile, causal, scale, sc);
  } else if (d == 128) {
    hipLaunchKernelGGL(dq_consolidate_kernel<128>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, parts,
                       reinterpret_cast<bf16*>(dq), N, row_stride, tile, causal, scale, sc);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dq_cast_blocks(const float* acc, void* dq, int64_t heads, int N, int row_stride, int d, float scale,
                                 StatusCopy sc, hipStream_t stream, const int* seqlens, int H) {
  const int64_t grid = heads * (row_stride / 32);
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (d == 64) {
    hipLaunchKernelGGL(dq_cast_blocks_kernel<64>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, acc,
                       reinterpret_cast<bf16*>(dq), N, row_stride, scale, seqlens, H, sc);
  } else if (d == 128) {
    hipLaunchKernelGGL(dq_cast_blocks_kernel<128>, dim3(static_cast<unsigned>(grid)), dim3(256), 0, stream, acc,
                       reinterpret_cast<bf16*>(dq), N, row_stride, scale, seqlens, H, sc);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_topology_probe(int* out, int grid, hipStream_t stream) {
  // Same LDS footprint class as the main kernel: one workgroup per CU.
  const int shmem = 83 * 1024;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(topology_probe_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, shmem);
  if (e != hipSuccess) return e;
  void* args[] = {&out};
  return launch_resident(reinterpret_cast<const void*>(topology_probe_kernel), grid, 64, shmem, args, stream);
}

}  // namespace dash
