// Main HIP kernel of the deterministic attention backward for gfx950 (MI355X).
//
// This file is compiled once per head dimension and workgroup size (DASH_MAIN_D =
// 64 or 128, DASH_MAIN_NW = 2 or 4 waves).
//
// Math (DASH paper, arXiv 2601.21824, section 2.1; "Writing an Attention Kernel",
// section "In the real world"): per (batch b, query head h, key/value head g):
//   P  = exp(s Q K^T - LSE)   (recomputed, masked entries 0)
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D)
//   (the dP accumulation starts from -D, so the accumulator holds dP - D)
//   dK = s dS^T Q,  dQ = s dS K
// Work decomposition (section 2.1, Fig. 1 left; section 3.1): a workgroup owns one
// KV tile at a time and keeps its dK/dV in registers while it visits Q tiles; the
// dQ partial sum of every visit goes to an fp32 accumulator in global memory,
// added in the order the schedule table fixes (ordered reduction, section 1) or
// with float atomics (the non-deterministic variant kept for comparison).
//
// CDNA4 mapping of the main kernel
// - One workgroup of NW waves per CU, persistent (one workgroup per CU, each reads
//   its task list from the schedule table). The workgroup learns its XCD from the
//   hardware (XCC_ID) and takes the next free slot of that XCD, so the table's CU
//   groups are CUs that share one L2.
// - KV tile = 32*NW rows; wave w owns KV rows [32w, 32w+32): their dK, dV (fp32) stay
//   in AGPR/VGPR accumulators for the whole item, and their K, V rows sit in
//   registers as MFMA B operands. Q tiles are visited in 64-row steps.
// - Q, dO (64 x d), -LSE*log2(e) and -D of the next step are copied global -> LDS with
//   global_load_lds_dwordx4 while the current step computes (double buffer).
// - All five contractions use v_mfma_f32_32x32x16_bf16. Operand layouts (A: lane
//   holds row lane%32, 8 consecutive k; B: column lane%32, 8 consecutive k; D:
//   column lane%32, rows 8*(r/4) + 4*(lane/32) + r%4):
//     S  = Q K^T    A = Q (ds_read_b128 from LDS), B = K (registers)
//     dP = dO V^T   A = dO (LDS), B = V (registers)
//     dV += P^T dO  A = P (registers, straight from the S accumulators), B = dO read
//                   with ds_read_b64_tr_b16 (LDS transpose read), rows permuted
//                   the same way as P's accumulator rows
//     dK += dS^T Q  likewise with dS and Q
//     dQ = dS K     A = dS via an LDS round trip (stored [kv][q], read transposed),
//                   B = K, read transposed from the item's K tile in LDS once per
//                   item and held in AGPRs with the accumulator
// - LDS tiles have one 16-byte pad chunk per row and operand rows are visited in a
//   permuted order (pi16), so that both the row reads (ds_read_b128) and the
//   transpose reads hit distinct banks with addresses "lane base + constant".
// - The dQ partial of a 64-row step is split over the waves by 32-column blocks;
//   every wave waits for and passes on its own turn (one semaphore per step and
//   wave), so the ordered reduction needs no workgroup barrier. The ordered variant's
//   fp32 accumulator is kept in the MFMA accumulator's order (kDqBlock), so a wave
//   reads and writes a block with four contiguous 1 KiB accesses at fixed offsets.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

#if !defined(DASH_MAIN_NW) || !defined(DASH_MAIN_D)
#error "DASH_MAIN_D (64 or 128) and DASH_MAIN_NW (2 or 4) must be defined"
#endif

namespace dash {

// ---------------------------------------------------------------------------------
// Main backward kernel.
// ---------------------------------------------------------------------------------
template <int D, int NW>
struct BwdCfg {
  static constexpr int BC = 32 * NW;    // KV (and Q) tile rows
  static constexpr int BQ = 64;         // Q rows per step
  static constexpr int SUBS = BC / BQ;  // steps per task
  static constexpr int NT = NW * 64;    // threads
  static constexpr int DB = D / 32;     // 32-column blocks of d
  static constexpr int DK = D / 16;     // k-steps over d
  static constexpr int KK = BC / 16;    // k-steps over the KV tile
  static constexpr int ST = TileGeom<D>::STRIDE;         // LDS row stride of Q, dO, K tiles
  static constexpr int NBLK = 2 * DB / NW;               // 32x32 dQ blocks per wave
  static constexpr int NKD = DB / NW > 1 ? DB / NW : 1;  // distinct d blocks per wave
  static constexpr int QT = BQ * ST;                     // bytes of one Q (or dO) tile
  static constexpr int DST = BC * kDsStride;             // bytes of one dS^T tile [BC][64]
  static constexpr int OFF_Q = 0;                        // 2 buffers
  static constexpr int OFF_DO = OFF_Q + 2 * QT;          // 2 buffers
  static constexpr int OFF_DS = OFF_DO + 2 * QT;         // 2 buffers
  static constexpr int OFF_K = OFF_DS + 2 * DST;         // K tile [BC][D]
  static constexpr int OFF_NL = OFF_K + BC * ST;         // 2 x 64 floats: -LSE*log2(e)
  static constexpr int OFF_DL = OFF_NL + 2 * 256;        // 2 x 64 floats: -D
  static constexpr int OFF_MISC = OFF_DL + 2 * 256;
  static constexpr int BYTES = OFF_MISC + 64;
  static_assert(NBLK >= 1 && NBLK * NW == 2 * DB, "dQ blocks must split evenly over waves");
  static_assert(SUBS >= 1 && SUBS * BQ == BC, "KV tile must be a multiple of 64 rows");
  static_assert(QT % 1024 == 0 && DST % 1024 == 0 && (BC * ST) % 1024 == 0, "1 KiB-aligned tiles");
};

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, 1)))
bwd_main_kernel(BwdParams p) {
  using C = BwdCfg<D, NW>;
  constexpr int BC = C::BC, BQ = C::BQ, SUBS = C::SUBS, DB = C::DB, DK = C::DK, KK = C::KK, ST = C::ST;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  LDS_AS int* sMisc = reinterpret_cast<LDS_AS int*>(smem + C::OFF_MISC);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int L16 = lane & 15;
  const int nb = (lane >> 4) & 1;

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

  PROF_DECL
  const int H = p.H, Hkv = p.Hkv, N = p.N;
  const bool cross = !p.xcd_local;
  bool failed = false;  // this wave gave up waiting (error reported); it keeps going without reducing
  // The schedule table is read-only for the whole launch: reading it through the
  // constant address space turns its uniform loads into scalar loads, which are
  // counted apart from the vector-memory queue that the global->LDS copies use.
  const CONST_AS int* worker_begin = (const CONST_AS int*)p.worker_begin;
  const CONST_AS Quad* items = (const CONST_AS Quad*)p.items;
  const CONST_AS Quad* tasks = (const CONST_AS Quad*)p.tasks;
  const int it_begin = worker_begin[worker];
  const int it_end = worker_begin[worker + 1];

  // Per-lane parts of the LDS addresses (the rest is a compile-time offset).
  // S, dP A operands: row pi(l32) (+32 qb), chunk hi (+2 ks).
  const int a_lane = pi16(l32) * ST + 16 * hi;
  // dV, dK B operands (transpose reads): row pi(16 hf + 8 s + 4 hi + j) - 16 hf - 2 s
  // = hi + 4 j, column 16 nb + 4 (L16 % 4) (+32 db).
  const int bt_lane = (hi + 4 * (L16 >> 2)) * ST + 2 * (16 * nb + 4 * (L16 & 3));
  // dQ contraction: KV row 16 kk + 2 hi + s + 4 j, column 16 nb + 4 (L16 % 4) (+32 qb or +32 db).
  const int kvrow_lane = 2 * hi + 4 * (L16 >> 2);
  const int col_lane2 = 2 * (16 * nb + 4 * (L16 & 3));
  const int ds_rd_lane = kvrow_lane * kDsStride + col_lane2;
  const int kd_lane = kvrow_lane * ST + col_lane2;
  // dS^T store: row 32 w + l32, bytes 8 hi (+16 t + 64 qb).
  const int ds_wr_lane = (32 * w + l32) * kDsStride + 8 * hi;

  LDS_AS char* sK = smem + C::OFF_K;
  TileCopy<D, BQ, NW> qcopy;  // copy plan of the Q and dO tiles
  qcopy.init(w, lane);
  const unsigned row_lane = static_cast<unsigned>(pi16(lane) * 4);  // LDS slot m <- row pi(m)

  for (int it = it_begin; it < it_end; ++it) {
    const Quad item = load_quad(items, it);
    const int b = item.x, g = item.y, kv_tile = item.z;
    const int t_begin = item.w, t_end = load_quad(items, it + 1).w;
    const int n_steps = (t_end - t_begin) * SUBS;
    const int kv0 = kv_tile * BC;
    const int64_t bg = static_cast<int64_t>(b) * Hkv + g;
    const bf16* Kg = p.k + bg * N * D;
    const bf16* Vg = p.v + bg * N * D;

    // Issues the global->LDS copies of step s (Q, dO, -LSE*log2e, -D) into buffer s & 1.
    auto issue_step = [&](int s) __attribute__((always_inline)) {
      const Quad task = load_quad(tasks, t_begin + s / SUBS);
      const int q0 = task.y * BC + (s % SUBS) * BQ;
      const int64_t bh = static_cast<int64_t>(b) * H + task.x;
      const int buf = s & 1;
      qcopy.issue(smem + C::OFF_Q + buf * C::QT, p.q + bh * N * D, q0, N, w);
      qcopy.issue(smem + C::OFF_DO + buf * C::QT, p.dO + bh * N * D, q0, N, w);
      // Row arrays are padded to the tile, so rows q0 .. q0+63 always exist.
      if (w == 0) dma4(p.nlse2 + bh * p.row_stride + q0, row_lane, smem + C::OFF_NL + buf * 256);
      if (w == 1) dma4(p.neg_delta + bh * p.row_stride + q0, row_lane, smem + C::OFF_DL + buf * 256);
    };

    // Item prologue: K tile to LDS, first step's tiles, K/V rows of this wave to registers.
    {
      TileCopy<D, BC, NW> kcopy;  // once per item: plan computed in place
      kcopy.init(w, lane);
      kcopy.issue(sK, Kg, kv0, N, w);
    }
    issue_step(0);
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
    floatx16 accK[DB], accV[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      accK[db] = floatx16{};
      accV[db] = floatx16{};
    }
    wait_mem_done();
    __syncthreads();
    if (kv0 + BC > N) {
      // Ragged KV tile: K rows past N become zero in LDS, so that the (unmasked,
      // finite) dS of those columns adds nothing to dQ. Their K/V registers are zero
      // already and their dK/dV rows are never stored.
      const int r0 = N - kv0;
      LDS_AS floatx4* z = reinterpret_cast<LDS_AS floatx4*>(sK + r0 * ST);
      for (int x = tid; x < (BC - r0) * ST / 16; x += C::NT) z[x] = floatx4{0.f, 0.f, 0.f, 0.f};
      __syncthreads();
    }
    const int kvcol = kv0 + 32 * w + l32;  // this lane's KV row in S, P, dP, dS
    // B operands of this wave's dQ blocks for the whole item: K^T of d block db_k(kd)
    // (kd < NKD), k-step kk covering KV rows 16 kk .. 16 kk + 15 in the order the dS
    // operand visits them (transpose reads of the K tile).
    auto db_k = [&](int kd) __attribute__((always_inline)) { return (w + NW * kd) % DB; };
    bf16x8 kT[C::NKD][KK];
#pragma unroll
    for (int kd = 0; kd < C::NKD; ++kd) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int koff = kd_lane + 16 * kk * ST + 64 * db_k(kd);
        kT[kd][kk] = join(lds_tr(sK, koff), lds_tr(sK, koff + ST));
      }
    }
    PROF_MARK(kProfItem);

    // Block t2 of this wave's dQ partial of step `ps` (its dS^T is in LDS buffer
    // ps & 1) = init + dS K, accumulated in place; accumulator row m of block qb is Q
    // row q0 + pi(32 qb + m). Block t2 uses d block db_k(t2 % NKD).
    auto dq_block = [&](int ps, int t2, floatx16& acc) __attribute__((always_inline)) {
      const LDS_AS char* sdSp = smem + C::OFF_DS + (ps & 1) * C::DST;
      const int qb = (w + NW * t2) / DB;
      const int kd = t2 % C::NKD;
      // A operand of k-step kk = dS (transpose reads of dS^T), loaded one k-step ahead.
      auto load = [&](int kk) __attribute__((always_inline)) -> bf16x8 {
        const int off = ds_rd_lane + 16 * kk * kDsStride + 64 * qb;
        return join(lds_tr(sdSp, off), lds_tr(sdSp, off + kDsStride));
      };
      bf16x8 a[2];
      a[0] = load(0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) a[(kk + 1) & 1] = load(kk + 1);
        mfma32_vab(acc, a[kk & 1], kT[kd][kk]);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_result_wait(acc);
    };

    // dQ addressing. Element r of this wave's block t2 at a step sits at row
    // q0 + 32 qb + 16 (t / 2) + 2 (t % 2) + hi + 4 e (r = 4 t + e) and column 32 db + l32
    // (the bf16 output and the atomic variant's row-major accumulator). In the ordered
    // variant's accumulator the block is number w + NW t2 of the step's 2 DB blocks and
    // elements 4 t .. 4 t + 3 of this lane sit at float 256 t + 4 lane (kDqBlock).
    auto blk_base = [&](int t2) __attribute__((always_inline)) {
      const int blk = w + NW * t2;
      return hi * D + (blk % DB) * 32 + l32;
    };
    auto row_const = [&](int t2, int r) __attribute__((always_inline)) {
      const int qb = (w + NW * t2) / DB;  // wave-uniform
      const int t = r >> 2, e = r & 3;
      return (32 * qb + 16 * (t >> 1) + 2 * (t & 1) + 4 * e) * D;
    };
    const int acc_lane = lane * 16;  // byte offset of this lane's first 4 floats in a block
    constexpr int kBlkBytes = kDqBlock * 4;

    // Reduction of step ps's dQ partial, in parts spread over the next step so that its
    // memory latency overlaps the step's work: (1) wait for the turn and issue the
    // accumulator loads, (2) per 32x32 block, the dQ MFMAs start from the loaded
    // accumulator and the sum is stored, (3) after the stores are acknowledged, pass
    // the turn on.
    struct Pending {
      int rank, last;
      int* sem;
      rsrc_t acc_rs;  // the step's 2 DB fp32 accumulator blocks
      rsrc_t dq_rs;   // bf16 dQ rows [q0, N) of (b, h)
      float* acc_g;   // atomic variant: accumulator row q0 (row-major)
      bool go;
    };
    auto reduce_begin = [&](int ps, floatx16 (&ld)[C::NBLK]) __attribute__((always_inline)) -> Pending {
      const Quad task = load_quad(tasks, t_begin + ps / SUBS);
      Pending pd;
      pd.rank = task.z;
      pd.last = task.w;
      const int q0s = task.y * BC + (ps % SUBS) * BQ;
      const int64_t bh = static_cast<int64_t>(b) * H + task.x;
      const int rows = N - q0s;  // may be <= 0 for a step past N
      // Accumulator rows are padded to the tile, so the step's blocks always exist.
      float* const acc_blk = p.dqacc + ((bh * (p.row_stride / 32) + q0s / 32) * DB) * kDqBlock;
      pd.acc_g = p.dqacc + (bh * p.row_stride + q0s) * D;
      pd.acc_rs = make_rsrc(acc_blk, 2 * DB * kBlkBytes);
      pd.dq_rs = make_rsrc(p.dq + bh * N * D + static_cast<int64_t>(q0s) * D, rows > 0 ? rows * D * 2 : 0);
      pd.sem = p.sem + bh * p.sem_stride + (task.y * SUBS + ps % SUBS) * 4 + w;
      pd.go = !failed;
      if (p.deterministic && pd.go && pd.rank > 0) {
        if (cross) {
          pd.go = wait_turn(pd.sem, pd.rank, p.err, p.timeout_ticks, true);
        } else {
          pd.go = wait_turn_local(pd.sem, pd.rank, p.err, p.timeout_ticks);
        }
        failed = !pd.go;
      }
      PROF_MARK(kProfWait);
      // Running sum so far; the first contributor (and the atomic variant) reads
      // through an empty descriptor, which returns zeros without touching memory.
      const bool add = p.deterministic && pd.go && pd.rank > 0;
      const rsrc_t lrs = make_rsrc(acc_blk, add ? 2 * DB * kBlkBytes : 0);
#pragma unroll
      for (int t2 = 0; t2 < C::NBLK; ++t2) {
        const int soff = (w + NW * t2) * kBlkBytes;  // wave-uniform block offset
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(lrs, acc_lane + 1024 * i, soff, kSC1);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned u = v[e];
            ld[t2][4 * i + e] = __builtin_bit_cast(float, u);
          }
        }
      }
      return pd;
    };
    auto reduce_store = [&](const Pending& pd, int t2, const floatx16& v) __attribute__((always_inline)) {
      if (!pd.go) return;
      if (!p.deterministic) {
        // Rows past N exist (padding) and are never output.
        float* dst = pd.acc_g + blk_base(t2);
#pragma unroll
        for (int r = 0; r < 16; ++r) atomicAdd(dst + row_const(t2, r), v[r]);
      } else if (pd.last) {
        const int vb = 2 * blk_base(t2);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const bf16 hv = static_cast<bf16>(v[r] * p.scale);
          __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, hv), pd.dq_rs,
                                                vb + 2 * row_const(t2, r), 0, 0);
        }
      } else {
        const int soff = (w + NW * t2) * kBlkBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // Element copied to a scalar first: a bit-cast of a vector element lvalue
            // reads the vector's first element.
            const float f = v[4 * i + e];
            x[e] = __builtin_bit_cast(unsigned, f);
          }
          __builtin_amdgcn_raw_buffer_store_b128(x, pd.acc_rs, acc_lane + 1024 * i, soff, 0);
        }
      }
    };
    // dQ blocks [t0, t1) of step ps (accumulated onto the loaded running sums) and
    // their stores.
    auto reduce_blocks = [&](int ps, const Pending& pd, floatx16 (&ld)[C::NBLK], int t0, int t1)
        __attribute__((always_inline)) {
#pragma unroll
      for (int t2 = t0; t2 < t1; ++t2) {
        dq_block(ps, t2, ld[t2]);
        reduce_store(pd, t2, ld[t2]);
      }
    };
    // Call after wait_mem_done(): this wave's accumulator stores are in the L2.
    auto reduce_signal = [&](const Pending& pd) __attribute__((always_inline)) {
      if (!p.deterministic || !pd.go || pd.last) return;
      if (cross) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      if (lane == 0) {
        if (cross)
          __hip_atomic_store(pd.sem, pd.rank + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        else
          __hip_atomic_store(pd.sem, pd.rank + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    };

    for (int s = 0; s < n_steps; ++s) {
      PROF_COUNT(kProfSteps);
      const int buf = s & 1;
      const Quad task = load_quad(tasks, t_begin + s / SUBS);
      const int j = task.y;
      const int q0 = j * BC + (s % SUBS) * BQ;

      // Previous step's reduction, part 1: wait for the turn, issue the accumulator
      // loads. The next step's copies go after them: waiting for those loads must not
      // wait for the copies (the vector-memory counter is in order).
      Pending pd;
      floatx16 ld[C::NBLK];
      const bool have_prev = s > 0;
      if (have_prev) pd = reduce_begin(s - 1, ld);
      constexpr int kBlkA = (C::NBLK + 1) / 2;  // dQ blocks reduced after the first S/dP block

      const LDS_AS char* sQ = smem + C::OFF_Q + buf * C::QT;
      const LDS_AS char* sdO = smem + C::OFF_DO + buf * C::QT;
      const LDS_AS char* sNL = smem + C::OFF_NL + buf * 256;
      const LDS_AS char* sDL = smem + C::OFF_DL + buf * 256;
      LDS_AS char* sdS = smem + C::OFF_DS + buf * C::DST;
      // Only the diagonal task of a causal mask needs a mask: rows past N have
      // -LSE*log2(e) = -inf (P = 0) and columns past N meet zero K rows in dQ.
      const bool diag = p.causal && j == kv_tile;
      // Causal diagonal (diagonal steps only): S = -inf, hence P = 0 and dS = 0, where the
      // key comes after the query, i.e. where pi(m) < kvcol - q0. Row of element r of
      // block qb: pi(m) = 32qb + 16(t/2) + 2(t%2) + 4e + hi (r = 4t + e).
      const int mask_thr = kvcol - q0 - hi;
      auto mask_diag = [&](int qb, floatx16& S) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = r >> 2, e = r & 3;
          if (32 * qb + 16 * (t >> 1) + 2 * (t & 1) + 4 * e < mask_thr) S[r] = -__builtin_inff();
        }
      };

      // The step body as an explicit software pipeline of "slots" separated by
      // scheduling barriers: each slot issues the LDS reads of the next slot's MFMA
      // operands, its own MFMAs, and a slice of the other 32-row block's softmax
      // (VALU), so that LDS latency and VALU work sit under the matrix cores.
      // Accumulator row m of a 32-row block qb is Q row pi(m).
      //
      // S = Q K^T and dP = dO V^T (block qb, this wave's 32 KV columns): A operands
      // from LDS, B = K/V rows in registers.
      auto sdp_off = [&](int qb, int ks) __attribute__((always_inline)) { return a_lane + 32 * qb * ST + 32 * ks; };
      // dV += P^T dO, dK += dS^T Q: iteration it = (hf, db); its B operands are the
      // transpose reads of dO and Q at Q/dO rows 16hf + hi + 4j (and + 2).
      auto bt_off = [&](int qb, int it) __attribute__((always_inline)) {
        return bt_lane + (32 * qb + 16 * (it / DB)) * ST + 64 * (it % DB);
      };
      auto load_bt = [&](int qb, int it, bf16x8& bo, bf16x8& bq) __attribute__((always_inline)) {
        const int off = bt_off(qb, it);
        bo = join(lds_tr(sdO, off), lds_tr(sdO, off + 2 * ST));
        bq = join(lds_tr(sQ, off), lds_tr(sQ, off + 2 * ST));
      };
      // Softmax of elements r0, r0+1 of block qb: P = exp2(s log2(e) S - LSE log2(e)),
      // dS = P (dP - D) (the dP accumulator already holds dP - D), both rounded to bf16
      // in pairs into Pw/dSw; after the fourth element of a row group t, dS^T of the
      // group goes to LDS ([kv][m]).
      auto softmax2 = [&](int qb, int r0, const floatx16& S, const floatx16& dP, const floatx4& nl, u32x4 (&Pw)[2],
                          u32x4 (&dSw)[2]) __attribute__((always_inline)) {
        const int e0 = r0 & 3;
        const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r0], p.scale_log2, nl[e0]));
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r0 + 1], p.scale_log2, nl[e0 + 1]));
        Pw[r0 >> 3][(r0 & 7) >> 1] = pack_bf16(p0, p1);
        dSw[r0 >> 3][(r0 & 7) >> 1] = pack_bf16(p0 * dP[r0], p1 * dP[r0 + 1]);
        if ((r0 & 3) == 2) {
          const int t = r0 >> 2;
          u32x2 v2;
          v2[0] = dSw[t >> 1][2 * (t & 1)];
          v2[1] = dSw[t >> 1][2 * (t & 1) + 1];
          *reinterpret_cast<LDS_AS u32x2*>(sdS + ds_wr_lane + 64 * qb + 16 * t) = v2;
        }
      };
      // -LSE*log2(e) of row group t (accumulator rows 8t + 4hi .. +3) of block qb.
      auto load_nl = [&](int qb, int t) __attribute__((always_inline)) -> floatx4 {
        return *reinterpret_cast<const LDS_AS floatx4*>(sNL + (qb * 32 + 8 * t + 4 * hi) * 4);
      };
      // -D of the 16 accumulator rows of block qb, in accumulator order: the start
      // value of the block's dP accumulation.
      auto load_negd = [&](int qb) __attribute__((always_inline)) -> floatx16 {
        floatx16 x;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const floatx4 d4 = *reinterpret_cast<const LDS_AS floatx4*>(sDL + (qb * 32 + 8 * t + 4 * hi) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[4 * t + e] = d4[e];
        }
        return x;
      };
      // Softmax of block qb spread over 8 slots (2 elements each); the row terms of
      // group t are loaded one slot before its first element (ring of 2).
      auto softmax_slot = [&](int qb, int slot, const floatx16& S, const floatx16& dP, floatx4 (&nlr)[2],
                              u32x4 (&Pw)[2], u32x4 (&dSw)[2]) __attribute__((always_inline)) {
        const int t = slot >> 1;
        softmax2(qb, 2 * slot, S, dP, nlr[t & 1], Pw, dSw);
        if ((slot & 1) && t + 1 < 4) nlr[(t + 1) & 1] = load_nl(qb, t + 1);
      };
#define SLOT() __builtin_amdgcn_sched_barrier(0)
      floatx16 S0 = {}, S1 = {};
      floatx16 dP0 = load_negd(0), dP1;
      u32x4 P0[2], dS0[2], P1[2], dS1[2];
      floatx4 nlr[2];
      bf16x8 aq[2], ad[2], bo[2], bq[2];
      static_assert(DK == 8 || DK == 4, "S/dP slots");
      constexpr int NIT = 2 * DB;  // dV/dK (hf, db) iterations, 2 MFMAs each
      // Block 0: S/dP (A operands one k-step ahead).
      aq[0] = lds_ld16(sQ, sdp_off(0, 0));
      ad[0] = lds_ld16(sdO, sdp_off(0, 0));
      SLOT();
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        if (ks + 1 < DK) {
          aq[(ks + 1) & 1] = lds_ld16(sQ, sdp_off(0, ks + 1));
          ad[(ks + 1) & 1] = lds_ld16(sdO, sdp_off(0, ks + 1));
        } else {
          aq[0] = lds_ld16(sQ, sdp_off(1, 0));
          ad[0] = lds_ld16(sdO, sdp_off(1, 0));
          nlr[0] = load_nl(0, 0);
        }
        if (ks == DK / 2) dP1 = load_negd(1);
        S0 = mfma32(aq[ks & 1], kreg[ks], S0);
        dP0 = mfma32(ad[ks & 1], vreg[ks], dP0);
        SLOT();
      }
      // Previous step's reduction, part 2 (first blocks): the loads have had block 0's
      // S/dP to arrive.
      if (have_prev) reduce_blocks(s - 1, pd, ld, 0, kBlkA);
      if (diag) mask_diag(0, S0);
      SLOT();
      // Block 1: S/dP, with block 0's softmax (8 slots of 2 elements over the DK k-steps).
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        if (ks + 1 < DK) {
          aq[(ks + 1) & 1] = lds_ld16(sQ, sdp_off(1, ks + 1));
          ad[(ks + 1) & 1] = lds_ld16(sdO, sdp_off(1, ks + 1));
        } else {
          load_bt(0, 0, bo[0], bq[0]);
        }
        S1 = mfma32(aq[ks & 1], kreg[ks], S1);
        dP1 = mfma32(ad[ks & 1], vreg[ks], dP1);
#pragma unroll
        for (int sl = (8 / DK) * ks; sl < (8 / DK) * (ks + 1); ++sl) softmax_slot(0, sl, S0, dP0, nlr, P0, dS0);
        if (ks + 1 == DK) nlr[0] = load_nl(1, 0);
        SLOT();
      }
      if (have_prev) {
        // Rest of the previous step's reduction; once its stores are acknowledged the
        // turn is passed on, half a step earlier than the step's end.
        reduce_blocks(s - 1, pd, ld, kBlkA, C::NBLK);
        wait_mem_done();
        reduce_signal(pd);
      }
      // The next step's copies: after every vector-memory load this step waits for.
      if (s + 1 < n_steps) issue_step(s + 1);
      if (diag) mask_diag(1, S1);
      SLOT();
      // Block 0: dV/dK (B operands one iteration ahead), with block 1's softmax.
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        if (it + 1 < NIT)
          load_bt(0, it + 1, bo[(it + 1) & 1], bq[(it + 1) & 1]);
        else
          load_bt(1, 0, bo[0], bq[0]);
        const int hf = it / DB, db = it % DB;
        mfma32_acc(accV[db], as_bf16x8(P0[hf]), bo[it & 1]);
        mfma32_acc(accK[db], as_bf16x8(dS0[hf]), bq[it & 1]);
#pragma unroll
        for (int sl = (8 / NIT) * it; sl < (8 / NIT) * (it + 1); ++sl) softmax_slot(1, sl, S1, dP1, nlr, P1, dS1);
        SLOT();
      }
      // Block 1: dV/dK.
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        if (it + 1 < NIT) load_bt(1, it + 1, bo[(it + 1) & 1], bq[(it + 1) & 1]);
        const int hf = it / DB, db = it % DB;
        mfma32_acc(accV[db], as_bf16x8(P1[hf]), bo[it & 1]);
        mfma32_acc(accK[db], as_bf16x8(dS1[hf]), bq[it & 1]);
        SLOT();
      }
#undef SLOT
      PROF_MARK(kProfBody);
      wait_mem_done();  // next step's tiles have landed
      PROF_MARK(kProfReduce);
      __syncthreads();  // dS^T of all waves and the next step's tiles are visible
      PROF_MARK(kProfBarrier);
    }
    // The item's last step: its dQ partial and reduction.
    {
      floatx16 ld[C::NBLK];
      const Pending pd = reduce_begin(n_steps - 1, ld);
      reduce_blocks(n_steps - 1, pd, ld, 0, C::NBLK);
      PROF_MARK(kProfDq);
      wait_mem_done();
      reduce_signal(pd);
      PROF_MARK(kProfReduce);
    }

    // Epilogue: dK = s dK, dV; bf16 stores of this wave's 32 KV rows.
    mfma_drain();
    bf16* dKg = p.dk + bg * N * D;
    bf16* dVg = p.dv + bg * N * D;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kvr = kv0 + 32 * w + 8 * (r >> 2) + 4 * hi + (r & 3);
        if (kvr < N) {
          const int off = kvr * D + db * 32 + l32;
          dKg[off] = static_cast<bf16>(accK[db][r] * p.scale);
          dVg[off] = static_cast<bf16>(accV[db][r]);
        }
      }
    }
    // Every wave is done with this item's LDS (K tile, last step's buffers) before
    // the next item's copies overwrite it.
    __syncthreads();
    PROF_MARK(kProfItem);
  }
  PROF_STORE(p, w, NW);
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

// One (d, waves) instantiation per translation unit, selected by DASH_MAIN_D and
// DASH_MAIN_NW, so that each can get its own code-generation flags.
#define DASH_CAT2(a, b, c, d) a##b##c##d
#define DASH_CAT(a, b, c, d) DASH_CAT2(a, b, c, d)
hipError_t DASH_CAT(launch_main_d, DASH_MAIN_D, _nw, DASH_MAIN_NW)(const BwdParams& prm, int grid, hipStream_t stream) {
  return launch_main_t<DASH_MAIN_D, DASH_MAIN_NW>(prm, grid, stream);
}

}  // namespace dash
