// HIP kernels of the deterministic attention backward for gfx950 (MI355X).
//
// Math (DASH paper, arXiv 2601.21824, section 2.1; "Writing an Attention Kernel",
// section "In the real world"): per (batch b, query head h, key/value head g):
//   P  = exp(s Q K^T - LSE)   (recomputed, masked entries 0)
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D)
//   dK = s dS^T Q,  dQ = s dS K
// Work decomposition (section 2.1, Fig. 1 left; section 3.1): a workgroup owns one
// KV tile at a time and keeps its dK/dV in registers while it visits Q tiles; the
// dQ partial sum of every visit goes to an fp32 accumulator in global memory,
// added in the order the schedule table fixes (ordered reduction, section 1) or
// with float atomics (the non-deterministic variant kept for comparison).
//
// CDNA4 mapping
// - One workgroup of NW waves (64 lanes each) per CU, persistent: the grid has one
//   workgroup per CU and each reads its task list from the schedule table. The
//   workgroup learns its XCD from the hardware (XCC_ID) and takes the next free
//   slot of that XCD, so the table's CU groups are the CUs of one L2 domain.
// - KV tile = 32*NW rows; wave w owns KV rows [32w, 32w+32) of it, so dK/dV of those
//   rows (32 x d fp32 each) stay in the wave's registers for the whole item.
// - Q tiles are visited in sub-tiles of 64 rows. Contractions use
//   v_mfma_f32_32x32x16_bf16 (A: lane holds row lane%32, 8 consecutive k;
//   B: column lane%32, 8 consecutive k; D: column lane%32, rows 8*(r/4)+4*(lane/32)+r%4).
// - S = Q K^T and dP = dO V^T take K and V from registers and Q, dO from LDS.
//   P and dS come out with one KV column per lane, which is exactly the A-operand
//   layout of dV += P^T dO and dK += dS^T Q (the 16 rows of a k-step are permuted
//   the same way on both operands). dQ = dS K needs dS with KV contiguous, so dS
//   goes through LDS once.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace dash {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ unsigned xcc_id() {
  // HW_REG_XCC_ID (hwreg 20), bits [3:0]: the XCD this wave runs on.
  return __builtin_amdgcn_s_getreg((20) | (0 << 6) | ((16 - 1) << 11)) & 0xfu;
}

__device__ __forceinline__ int load_flag_sys(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ void raise_error(int* err, int code) {
  int expected = 0;
  __hip_atomic_compare_exchange_strong(err, &expected, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_SYSTEM);
}

// Spin until *sem == want. Returns false if the wait timed out or another
// workgroup reported an error (the caller then stops; no wait is unbounded).
// The semaphore is read with agent-scope loads, which skip the CU's L1 and are
// served by the L2. With `cross_xcd` the contributors of one dQ tile may sit on
// different XCDs, whose L2s are not coherent with each other: then an agent-scope
// acquire fence (L1/L2 invalidate) follows the wait.
__device__ bool wait_turn(const int* sem, int want, int* err, long long timeout_ticks, bool cross_xcd) {
  const long long t0 = wall_clock64();
  int iter = 0;
  while (true) {
    const int s = __hip_atomic_load(sem, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (s == want) break;
    if ((++iter & 31) == 0) {
      if (load_flag_sys(err) != 0) return false;
      if (wall_clock64() - t0 > timeout_ticks) {
        raise_error(err, kErrTimeout);
        return false;
      }
    }
    __builtin_amdgcn_s_sleep(1);
  }
  if (cross_xcd) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return true;
}

// Waits until every global store this wave issued has been acknowledged by the
// L2 (s_waitcnt vmcnt(0)); the signal fences keep the compiler from moving
// memory operations across it.
__device__ __forceinline__ void wait_stores_done() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ---------------------------------------------------------------------------------
// Preprocess: D[row] = sum_e dO[row, e] * O[row, e] in fp32 with a fixed reduction
// tree; clears the ordering semaphores and the XCD slot counters; for the atomic
// variant also clears the fp32 dQ accumulator.
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
    if (part == 0) p.delta[row] = acc;
  }
  for (int64_t x = tid; x < p.sem_count; x += nthreads) p.sem[x] = 0;
  for (int64_t x = tid; x < p.ctr_count; x += nthreads) p.ctr[x] = 0;
  if (p.dqacc_zero) {
    floatx4* z = reinterpret_cast<floatx4*>(p.dqacc_zero);
    const floatx4 zero = {0.f, 0.f, 0.f, 0.f};
    for (int64_t x = tid; x < p.zero_count / 4; x += nthreads) z[x] = zero;
  }
}

// dQ = bf16(s * dQacc), for the atomic variant (the ordered variant writes dQ from
// the last contributor of each tile).
__global__ void __launch_bounds__(256) dq_cast_kernel(const float* __restrict__ acc, bf16* __restrict__ dq,
                                                      int64_t count, float scale) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t nthreads = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t x = tid; x < count / 4; x += nthreads) {
    const floatx4 a = reinterpret_cast<const floatx4*>(acc)[x];
    bf16x4 r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = static_cast<bf16>(a[e] * scale);
    reinterpret_cast<bf16x4*>(dq)[x] = r;
  }
}

// Records the XCD of every workgroup of a one-workgroup-per-CU grid.
__global__ void __launch_bounds__(64) topology_probe_kernel(int* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = static_cast<int>(xcc_id());
}

// ---------------------------------------------------------------------------------
// Main backward kernel.
// ---------------------------------------------------------------------------------
template <int D, int NW>
struct BwdCfg {
  static constexpr int BC = 32 * NW;   // KV (and Q) tile rows
  static constexpr int BR = 64;        // Q sub-tile rows
  static constexpr int QB = BR / 32;   // 32-row blocks per sub-tile
  static constexpr int DB = D / 32;    // 32-column blocks of d
  static constexpr int DK = D / 16;    // k-steps over d
  static constexpr int SUBS = BC / BR; // sub-tiles per Q tile
  static constexpr int NT = NW * 64;   // threads
  static constexpr int NBLK = QB * DB / NW;  // dQ output blocks per wave
  static constexpr int LDQ = D + 8;    // row stride of Q, dO in LDS (elements)
  static constexpr int LDT = BR + 8;   // row stride of Q^T, dO^T
  static constexpr int LDS = BC + 8;   // row stride of dS [q][kv]
  static constexpr int LDK = BC + 8;   // row stride of K^T [d][kv]
  static constexpr int OFF_Q = 0;
  static constexpr int OFF_DO = OFF_Q + BR * LDQ * 2;
  static constexpr int OFF_QT = OFF_DO + BR * LDQ * 2;
  static constexpr int OFF_DOT = OFF_QT + D * LDT * 2;
  static constexpr int OFF_DS = OFF_DOT + D * LDT * 2;
  static constexpr int OFF_KT = OFF_DS + BR * LDS * 2;
  static constexpr int OFF_L = OFF_KT + D * LDK * 2;
  static constexpr int OFF_DL = OFF_L + BR * 4;
  static constexpr int OFF_MISC = OFF_DL + BR * 4;
  static constexpr int BYTES = OFF_MISC + 64;
  static_assert(NBLK >= 1 && NBLK * NW == QB * DB, "dQ blocks must split evenly over waves");
};

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_main_kernel(BwdParams p) {
  using C = BwdCfg<D, NW>;
  constexpr int BC = C::BC, BR = C::BR, QB = C::QB, DB = C::DB, DK = C::DK, SUBS = C::SUBS, NT = C::NT;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16* sQ = reinterpret_cast<bf16*>(smem + C::OFF_Q);
  bf16* sdO = reinterpret_cast<bf16*>(smem + C::OFF_DO);
  bf16* sQt = reinterpret_cast<bf16*>(smem + C::OFF_QT);
  bf16* sdOt = reinterpret_cast<bf16*>(smem + C::OFF_DOT);
  bf16* sdS = reinterpret_cast<bf16*>(smem + C::OFF_DS);
  bf16* sKt = reinterpret_cast<bf16*>(smem + C::OFF_KT);
  float* sL = reinterpret_cast<float*>(smem + C::OFF_L);
  float* sDl = reinterpret_cast<float*>(smem + C::OFF_DL);
  int* sMisc = reinterpret_cast<int*>(smem + C::OFF_MISC);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Worker slot: XCD from hardware, slot = arrival order within that XCD.
  if (tid == 0) {
    unsigned x = (p.num_xcd == 1) ? 0u : xcc_id();
    int v = -1;
    if (x < static_cast<unsigned>(p.num_xcd)) {
      const int slot = atomicAdd(p.ctr + x * 64, 1);
      if (slot < p.cus_per_xcd) v = static_cast<int>(x) * p.cus_per_xcd + slot;
    }
    if (v < 0) raise_error(p.err, kErrPlacement);
    sMisc[0] = v;
  }
  __syncthreads();
  const int worker = sMisc[0];
  if (worker < 0) return;

  const int H = p.H, Hkv = p.Hkv, N = p.N;
  const int it_begin = p.worker_begin[worker];
  const int it_end = p.worker_begin[worker + 1];

  for (int it = it_begin; it < it_end; ++it) {
    const int4 item = p.items[it];
    const int b = item.x, g = item.y, kv_tile = item.z;
    const int t_begin = item.w, t_end = p.items[it + 1].w;
    const int kv0 = kv_tile * BC;
    const bf16* Kg = p.k + (static_cast<int64_t>(b) * Hkv + g) * N * D;
    const bf16* Vg = p.v + (static_cast<int64_t>(b) * Hkv + g) * N * D;

    // K and V rows of this wave as MFMA B operands (column = KV row, k = d).
    bf16x8 kreg[DK], vreg[DK];
    {
      const int kvr = kv0 + 32 * w + l32;
      const bool ok = kvr < N;
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        bf16x8 kz = {}, vz = {};
        if (ok) {
          kz = *reinterpret_cast<const bf16x8*>(Kg + static_cast<int64_t>(kvr) * D + ks * 16 + 8 * hi);
          vz = *reinterpret_cast<const bf16x8*>(Vg + static_cast<int64_t>(kvr) * D + ks * 16 + 8 * hi);
        }
        kreg[ks] = kz;
        vreg[ks] = vz;
      }
    }
    // K^T of the whole tile in LDS ([d][kv]) for dQ = dS K.
    for (int c = tid; c < BC * D / 8; c += NT) {
      const int row = c / (D / 8);
      const int col = (c % (D / 8)) * 8;
      bf16x8 val = {};
      if (kv0 + row < N) val = *reinterpret_cast<const bf16x8*>(Kg + static_cast<int64_t>(kv0 + row) * D + col);
#pragma unroll
      for (int e = 0; e < 8; ++e) sKt[(col + e) * C::LDK + row] = val[e];
    }

    floatx16 accK[DB], accV[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      accK[db] = floatx16{};
      accV[db] = floatx16{};
    }

    for (int t = t_begin; t < t_end; ++t) {
      const int4 task = p.tasks[t];
      const int h = task.x, j = task.y, rank = task.z, last = task.w;
      const int64_t bh = static_cast<int64_t>(b) * H + h;
      const bf16* Qg = p.q + bh * N * D;
      const bf16* dOg = p.dO + bh * N * D;

      for (int sub = 0; sub < SUBS; ++sub) {
        const int q0 = j * BC + sub * BR;
        // Stage Q, dO (row-major and transposed), LSE (base 2) and D of the sub-tile.
        for (int c = tid; c < BR * D / 8; c += NT) {
          const int row = c / (D / 8);
          const int col = (c % (D / 8)) * 8;
          bf16x8 qv = {}, dv = {};
          if (q0 + row < N) {
            qv = *reinterpret_cast<const bf16x8*>(Qg + static_cast<int64_t>(q0 + row) * D + col);
            dv = *reinterpret_cast<const bf16x8*>(dOg + static_cast<int64_t>(q0 + row) * D + col);
          }
          *reinterpret_cast<bf16x8*>(sQ + row * C::LDQ + col) = qv;
          *reinterpret_cast<bf16x8*>(sdO + row * C::LDQ + col) = dv;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            sQt[(col + e) * C::LDT + row] = qv[e];
            sdOt[(col + e) * C::LDT + row] = dv[e];
          }
        }
        for (int r = tid; r < BR; r += NT) {
          const int qr = q0 + r;
          sL[r] = (qr < N) ? p.lse[bh * N + qr] * kLog2e : __builtin_inff();
          sDl[r] = (qr < N) ? p.delta[bh * N + qr] : 0.f;
        }
        __syncthreads();

        // S = Q K^T and dP = dO V^T for this wave's 32 KV columns.
        floatx16 S[QB], dP[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          S[qb] = floatx16{};
          dP[qb] = floatx16{};
#pragma unroll
          for (int ks = 0; ks < DK; ++ks) {
            const int off = (qb * 32 + l32) * C::LDQ + ks * 16 + 8 * hi;
            const bf16x8 aq = *reinterpret_cast<const bf16x8*>(sQ + off);
            const bf16x8 ad = *reinterpret_cast<const bf16x8*>(sdO + off);
            S[qb] = mfma32(aq, kreg[ks], S[qb]);
            dP[qb] = mfma32(ad, vreg[ks], dP[qb]);
          }
        }

        // P = exp2(s log2(e) S - LSE log2(e)), dS = P (dP - D); rounded to bf16.
        bf16x8 Pb[QB][2], dSb[QB][2];
        const int kvg = kv0 + 32 * w + l32;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ql = qb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            const int qg = q0 + ql;
            float pr = __builtin_amdgcn_exp2f(S[qb][r] * p.scale_log2 - sL[ql]);
            if ((p.causal && kvg > qg) || kvg >= N) pr = 0.f;
            const float ds = pr * (dP[qb][r] - sDl[ql]);
            Pb[qb][r >> 3][r & 7] = static_cast<bf16>(pr);
            dSb[qb][r >> 3][r & 7] = static_cast<bf16>(ds);
          }
        }

        // dV += P^T dO, dK += dS^T Q (A from registers, B = dO^T / Q^T from LDS).
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int dcol = db * 32 + l32;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const int qbase = qb * 32 + 16 * hf + 4 * hi;
              const bf16x4 o0 = *reinterpret_cast<const bf16x4*>(sdOt + dcol * C::LDT + qbase);
              const bf16x4 o1 = *reinterpret_cast<const bf16x4*>(sdOt + dcol * C::LDT + qbase + 8);
              const bf16x4 q0v = *reinterpret_cast<const bf16x4*>(sQt + dcol * C::LDT + qbase);
              const bf16x4 q1v = *reinterpret_cast<const bf16x4*>(sQt + dcol * C::LDT + qbase + 8);
              const bf16x8 bo = __builtin_shufflevector(o0, o1, 0, 1, 2, 3, 4, 5, 6, 7);
              const bf16x8 bq = __builtin_shufflevector(q0v, q1v, 0, 1, 2, 3, 4, 5, 6, 7);
              accV[db] = mfma32(Pb[qb][hf], bo, accV[db]);
              accK[db] = mfma32(dSb[qb][hf], bq, accK[db]);
            }
          }
        }

        // dS to LDS as [q][kv] for dQ = dS K.
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ql = qb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            sdS[ql * C::LDS + 32 * w + l32] = dSb[qb][r >> 3][r & 7];
          }
        }
        __syncthreads();

        floatx16 dq[C::NBLK];
#pragma unroll
        for (int t2 = 0; t2 < C::NBLK; ++t2) {
          const int blk = w + NW * t2;
          const int qb = blk / DB, db = blk % DB;
          floatx16 acc = {};
#pragma unroll
          for (int kk = 0; kk < BC / 16; ++kk) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(sdS + (qb * 32 + l32) * C::LDS + kk * 16 + 8 * hi);
            const bf16x8 bk = *reinterpret_cast<const bf16x8*>(sKt + (db * 32 + l32) * C::LDK + kk * 16 + 8 * hi);
            acc = mfma32(a, bk, acc);
          }
          dq[t2] = acc;
        }

        // Reduction of this sub-tile's dQ partial sum into dQ tile (b, h, j, sub).
        float* acc_g = p.dqacc + bh * N * D;
        if (p.deterministic) {
          // Ordered reduction. XCD-local tables (every contributor of this dQ tile on
          // one XCD): the XCD's L2 is the point of coherence, so the accumulator is
          // read with L1-bypassing agent-scope loads, written with plain
          // (write-through) stores, and the turn is passed on once all stores are
          // acknowledged. Otherwise agent-scope release/acquire fences are used.
          const bool cross = !p.xcd_local;
          int* sem = p.sem + bh * p.sem_stride + j * SUBS + sub;
          if (rank > 0) {
            if (tid == 0) sMisc[1] = wait_turn(sem, rank, p.err, p.timeout_ticks, cross) ? 1 : 0;
            __syncthreads();
            if (!sMisc[1]) return;
            if (cross) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
          }
#pragma unroll
          for (int t2 = 0; t2 < C::NBLK; ++t2) {
            const int blk = w + NW * t2;
            const int qb = blk / DB, db = blk % DB;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int qg = q0 + qb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              if (qg < N) {
                const int64_t off = static_cast<int64_t>(qg) * D + db * 32 + l32;
                float val = dq[t2][r];
                if (rank > 0) val = __hip_atomic_load(acc_g + off, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + val;
                if (last)
                  p.dq[bh * N * D + off] = static_cast<bf16>(val * p.scale);
                else
                  acc_g[off] = val;
              }
            }
          }
          if (!last) {
            if (cross)
              __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            else
              wait_stores_done();
            __syncthreads();
            if (tid == 0) {
              if (cross)
                __hip_atomic_store(sem, rank + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
              else
                __hip_atomic_store(sem, rank + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
          }
        } else {
#pragma unroll
          for (int t2 = 0; t2 < C::NBLK; ++t2) {
            const int blk = w + NW * t2;
            const int qb = blk / DB, db = blk % DB;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int qg = q0 + qb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              if (qg < N) atomicAdd(acc_g + static_cast<int64_t>(qg) * D + db * 32 + l32, dq[t2][r]);
            }
          }
        }
        __syncthreads();
      }
    }

    // Epilogue: dK = s dK, dV; bf16 stores of this wave's 32 KV rows.
    bf16* dKg = p.dk + (static_cast<int64_t>(b) * Hkv + g) * N * D;
    bf16* dVg = p.dv + (static_cast<int64_t>(b) * Hkv + g) * N * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kvr = kv0 + 32 * w + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (kvr < N) {
          const int64_t off = static_cast<int64_t>(kvr) * D + db * 32 + l32;
          dKg[off] = static_cast<bf16>(accK[db][r] * p.scale);
          dVg[off] = static_cast<bf16>(accV[db][r]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------
template <int D, int NW>
static hipError_t launch_main_t(const BwdParams& prm, int grid, hipStream_t stream) {
  using C = BwdCfg<D, NW>;
  // At least 81 KiB of LDS so that exactly one workgroup fits on a CU.
  const int shmem = C::BYTES > 83 * 1024 ? C::BYTES : 83 * 1024;
  auto fn = bwd_main_kernel<D, NW>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, shmem);
  if (e != hipSuccess) return e;
  BwdParams local = prm;
  void* args[] = {&local};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(fn), dim3(grid), dim3(NW * 64), args,
                                    shmem, stream);
}

hipError_t launch_main(const BwdParams& prm, int d, int nw, int grid, hipStream_t stream) {
  if (d == 64 && nw == 2) return launch_main_t<64, 2>(prm, grid, stream);
  if (d == 64 && nw == 4) return launch_main_t<64, 4>(prm, grid, stream);
  if (d == 128 && nw == 2) return launch_main_t<128, 2>(prm, grid, stream);
  if (d == 128 && nw == 4) return launch_main_t<128, 4>(prm, grid, stream);
  return hipErrorInvalidValue;
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

hipError_t launch_dq_cast(const float* acc, void* dq, int64_t count, float scale, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(dq_cast_kernel, dim3(grid), dim3(256), 0, stream, acc, reinterpret_cast<bf16*>(dq), count,
                     scale);
  return hipGetLastError();
}

hipError_t launch_topology_probe(int* out, int grid, hipStream_t stream) {
  // Same LDS footprint class as the main kernel: one workgroup per CU.
  const int shmem = 83 * 1024;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(topology_probe_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, shmem);
  if (e != hipSuccess) return e;
  void* args[] = {&out};
  return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(topology_probe_kernel), dim3(grid), dim3(64),
                                    args, shmem, stream);
}

int main_kernel_lds_bytes(int d, int nw) {
  int b = 0;
  if (d == 64 && nw == 2) b = BwdCfg<64, 2>::BYTES;
  if (d == 64 && nw == 4) b = BwdCfg<64, 4>::BYTES;
  if (d == 128 && nw == 2) b = BwdCfg<128, 2>::BYTES;
  if (d == 128 && nw == 4) b = BwdCfg<128, 4>::BYTES;
  return b > 83 * 1024 ? b : 83 * 1024;
}

}  // namespace dash
