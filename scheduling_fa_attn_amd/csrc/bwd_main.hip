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
// with float atomics (the non-deterministic variant kept for comparison). A separate
// kernel casts the final sums to bf16 dQ. For the two-pass variant (the alternative
// design of section 5) the dQ work is compiled out and dQ comes from its own pass.
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
//     S  = Q K^T    A = Q (ds_read_b128 from LDS), B = K (AGPRs, loaded per item)
//     dP = dO V^T   A = dO (LDS), B = V (AGPRs)
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
// - The step is an explicit software pipeline (one wave per SIMD, so the wave itself
//   must overlap MFMAs with LDS latency, softmax VALU and memory traffic); its hot path
//   has no per-store or per-copy branches (empty buffer descriptors drop the stores
//   that must not happen) and its bookkeeping comes from a per-step record read two
//   steps ahead.
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

// DET: ordered reduction (p.deterministic != 0) or float atomics; one kernel each, so
// that neither carries the other's code and registers. CROSS (ordered reduction only):
// the contributors of one dQ tile may sit on different XCDs, whose L2s are not coherent
// with each other, so the running sums and turns go through device-scope loads and
// stores (no whole-L2 write-back or invalidate); otherwise every chain stays inside one
// XCD's L2. NODQ (with !DET): dK and dV
// only, no dQ work at all (the two-pass variant computes dQ in a separate kernel).
template <int D, int NW, bool DET, bool CROSS, bool NODQ, bool PART>
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
  // Rows of batch b: N, or seqlens[b] <= N for variable-length batches (N stays the row
  // stride of every tensor; rows past a batch's length are padding, never read as data).
  const CONST_AS int* seqlens = (const CONST_AS int*)p.seqlens;
  auto len_of = [&](int b) __attribute__((always_inline)) { return p.seqlens ? seqlens[b] : N; };
  constexpr bool cross = CROSS;
  static_assert(DET || !CROSS, "device-scope chains exist only in the ordered reduction");
  static_assert(!(DET && NODQ), "the ordered reduction reduces dQ");
  static_assert(!PART || (DET && !CROSS), "per-tile partials: stores into slots, no chains");
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

  // Copies of an item's tiles, issued while the previous item finishes (its last step
  // and its last reduction), so that an item starts with its data in LDS:
  //  - K (BC x D) -> the K tile; it is read only by the item's prologue;
  //  - V (BC x D) -> the Q and dO areas of the buffer its step 0 does not use (rows
  //    64 h .. 64 h + 63 in area h), free from the end of the previous item's last step
  //    until the item's step 0 issues step 1's copies;
  //  - the first step's Q, dO, -LSE*log2e, -D -> the buffer of its step 0 (with the
  //    previous item's last step copies, below).
  // Buffers alternate by step across items: an item's step s uses buffer (par0 + s) & 1.
  auto issue_kv = [&](int it2, int par0) __attribute__((always_inline)) {
    const Quad item2 = load_quad(items, it2);
    const int64_t bg2 = static_cast<int64_t>(item2.x) * Hkv + item2.y;
    const int kv02 = item2.z * BC;
    const int nrow2 = len_of(item2.x);
    TileCopy<D, BC, NW> kcopy;  // plan computed in place
    kcopy.init(w, lane);
    kcopy.issue(sK, p.k + bg2 * N * D, kv02, nrow2, w);
#pragma unroll
    for (int hh = 0; hh < BC / BQ; ++hh)
      qcopy.issue(smem + (hh == 0 ? C::OFF_Q : C::OFF_DO) + (par0 ^ 1) * C::QT, p.v + bg2 * N * D, kv02 + BQ * hh, nrow2,
                  w);
  };
  auto issue_first_step = [&](int it2, int par0) __attribute__((always_inline)) {
    const Quad item2 = load_quad(items, it2);
    const Quad task = load_quad(tasks, item2.w);
    const int q0 = task.y * BC;
    const int64_t bh = static_cast<int64_t>(item2.x) * H + task.x;
    const int nrow2 = len_of(item2.x);
    qcopy.issue(smem + C::OFF_Q + par0 * C::QT, p.q + bh * N * D, q0, nrow2, w);
    qcopy.issue(smem + C::OFF_DO + par0 * C::QT, p.dO + bh * N * D, q0, nrow2, w);
    // Row arrays are padded to the tile, so rows q0 .. q0+63 always exist.
    if (w == 0) dma4(p.nlse2 + bh * p.row_stride + q0, row_lane, smem + C::OFF_NL + par0 * 256);
    if (w == 1) dma4(p.neg_delta + bh * p.row_stride + q0, row_lane, smem + C::OFF_DL + par0 * 256);
  };
  int par0 = 0;  // buffer of the current item's step 0
  // Step records (p.steps: {b * H + h, first Q row, rank, last} per 64-row step) of the
  // current and the next step, carried across steps and items (a worker's steps are
  // contiguous in the stream); the record two steps ahead is read during a step and
  // taken over at its end, so no step waits for a table read.
  const CONST_AS Quad* steps = (const CONST_AS Quad*)p.steps;
  Quad rec_cur = {0, 0, 0, 0}, rec_nxt = {0, 0, 0, 0};
  if (it_begin < it_end) {
    issue_kv(it_begin, par0);
    issue_first_step(it_begin, par0);
    const int gs0 = load_quad(items, it_begin).w * SUBS;
    rec_cur = load_quad(steps, gs0);
    rec_nxt = load_quad(steps, gs0 + 1);
  }

  for (int it = it_begin; it < it_end; ++it) {
    const Quad item = load_quad(items, it);
    const int kv_tile = item.z;
    const int t_begin = item.w, t_end = load_quad(items, it + 1).w;
    const int n_steps = (t_end - t_begin) * SUBS;
    const int kv0 = kv_tile * BC;
    const int64_t bg = static_cast<int64_t>(item.x) * Hkv + item.y;
    const int nrow = len_of(item.x);  // rows of this item's batch
    const bool has_next = it + 1 < it_end;

    // Item prologue: the item's tiles (issued before) have landed; K and V rows of this
    // wave to AGPRs, dK and dV accumulators zeroed.
    wait_mem_done();
    __syncthreads();
    if (kv0 + BC > nrow) {
      // Ragged KV tile: K rows past the batch's length become zero in LDS, so that the
      // (unmasked, finite) dS of those columns adds nothing to dQ. Their dK/dV rows are
      // never stored; their K/V operands (copies of the last row) only feed those rows.
      const int r0 = nrow - kv0;
      LDS_AS floatx4* z = reinterpret_cast<LDS_AS floatx4*>(sK + r0 * ST);
      for (int x = tid; x < (BC - r0) * ST / 16; x += C::NT) z[x] = floatx4{0.f, 0.f, 0.f, 0.f};
      __syncthreads();
    }
    bf16x8 kreg[DK], vreg[DK];
    {
      // Row 32 w + l32 of the tile; the B operand of k-step ks holds its d columns
      // 16 ks + 8 hi .. + 7.
      const int r = 32 * w + l32;
      const LDS_AS char* vrow = smem + (r < BQ ? C::OFF_Q : C::OFF_DO) + (par0 ^ 1) * C::QT + (r % BQ) * ST;
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        kreg[ks] = to_agpr(lds_ld16(sK, r * ST + 32 * ks + 16 * hi));
        vreg[ks] = to_agpr(lds_ld16(vrow, 32 * ks + 16 * hi));
      }
    }
    floatx16 accK[DB], accV[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      accK[db] = floatx16{};
      accV[db] = floatx16{};
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
        kT[kd][kk] = NODQ ? bf16x8{} : to_agpr(join(lds_tr(sK, koff), lds_tr(sK, koff + ST)));
      }
    }
    // Every wave has its V rows before step 0 issues step 1's copies into buffer 1.
    __syncthreads();
    PROF_MARK(kProfPro);

    // The dQ MFMAs start from the loaded running sum, except in the atomic variant and in
    // replay builds, which start from zero: then the first k-step uses a literal 0 as its
    // accumulator input, so that no VALU instruction writes the accumulator right before
    // an inline MFMA reads it.
#ifdef DASH_REPLAY
    constexpr bool kZeroStart = true;
#else
    constexpr bool kZeroStart = !DET || PART;
#endif
    auto dq_mma = [&](floatx16& acc, int kk, const bf16x8& a, const bf16x8& b) __attribute__((always_inline)) {
      if (kZeroStart && kk == 0)
        mfma32_vab_zero(acc, a, b);
      else
        mfma32_vab(acc, a, b);
    };
    // Block t2 of this wave's dQ partial of step `ps` (its dS^T is in LDS buffer
    // (par0 + ps) & 1) = init + dS K, accumulated in place; accumulator row m of block qb is Q
    // row q0 + pi(32 qb + m). Block t2 uses d block db_k(t2 % NKD).
    auto dq_block = [&](int ps, int t2, floatx16& acc) __attribute__((always_inline)) {
      if (NODQ) return;
      const LDS_AS char* sdSp = smem + C::OFF_DS + ((par0 + ps) & 1) * C::DST;
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
        dq_mma(acc, kk, a[kk & 1], kT[kd][kk]);
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
    constexpr int kBlkBytes = kDqBlock * 4;
    // Ordered variant: byte offset of this lane's first 4 floats in block w + NW t2 of a
    // step's 2 DB accumulator blocks; part i (floats 256 i ..) adds the immediate 1024 i.
    int acc_off[C::NBLK];
#pragma unroll
    for (int t2 = 0; t2 < C::NBLK; ++t2) acc_off[t2] = lane * 16 + (w + NW * t2) * kBlkBytes;

    // Ordered reduction of step ps's dQ partial (DASH paper, section 3.1: contributions
    // to one dQ tile are added in the order the schedule table ranks them). Its parts
    // are spread so that memory latency overlaps other work: (1) the bookkeeping and a
    // poll of the turn during the last MFMA phase of step ps, (2) once the turn has come,
    // the running-sum loads (then or, failing that, at the start of step ps + 1, after a
    // blocking wait), (3) the dQ MFMAs, which start from the loaded running sum, inside
    // the S/dP slots of step ps + 1, (4) the stores, spread over the following slots,
    // (5) after the stores are acknowledged, the turn is passed on.
    // Every contributor, the last one included, stores its running sum (the final sums are
    // cast to bf16 dQ by a separate kernel), so that every step runs the same code. Stores
    // that must not happen (a contribution whose wait failed, step 0's missing previous
    // partial) go through an empty descriptor, which drops them: the stores spread over
    // the step's slots need no branch.
    struct Pending {
      int rank, last;
      int* sem;
      float* acc_blk; // the step's first fp32 accumulator block
      rsrc_t acc_rs;  // fp32 stores: the step's 2 DB accumulator blocks (atomic variant: its
                      // rows q0 .. q0 + 63 of the row-major accumulator); empty if none
      bool go;
#ifdef DASH_REPLAY
      float* dump;    // replay builds: dump slot of the step's first block at this rank
#endif
    };
    // `rec` is the step's record: {b * H + h, first Q row, rank, last}.
    auto reduce_prepare = [&](const Quad& rec) __attribute__((always_inline)) -> Pending {
      Pending pd;
      pd.rank = rec.z;
      pd.last = rec.w;
      const int q0s = rec.y;
      const int64_t bh = rec.x;
      // Accumulator rows are padded to the tile, so the step's blocks always exist.
      if (PART) {
        // Per-tile partials: the step's own slot, (b * H + h, step, rank), in the compact
        // layout described at kDqBlock.
        pd.acc_blk = p.dqacc + partial_slot(bh, q0s, pd.rank, p.row_stride / BC, BC, p.causal) * (2 * DB) * kDqBlock;
      } else {
        pd.acc_blk = p.dqacc + ((bh * (p.row_stride / 32) + q0s / 32) * DB) * kDqBlock;
      }
      pd.go = !failed;
      pd.acc_rs = DET ? make_rsrc(pd.acc_blk, pd.go ? 2 * DB * kBlkBytes : 0)
                      : make_rsrc(p.dqacc + (bh * p.row_stride + q0s) * D, pd.go ? 64 * D * 4 : 0);
      pd.sem = p.sem + bh * p.sem_stride + (q0s / BQ) * kSemPerStep + w;
#ifdef DASH_REPLAY
      // Dump layout: [b*H + h][64-row step][dQ block (2 DB)][rank][kDqBlock floats].
      pd.dump = p.replay ? p.replay + (((bh * (p.row_stride / BQ) + q0s / BQ) * (2 * DB)) * p.replay_ranks + pd.rank) *
                                          static_cast<int64_t>(kDqBlock)
                         : nullptr;
#endif
      return pd;
    };
    // Does this contribution have to wait for its turn at all?
    auto reduce_needs_turn = [&](const Pending& pd) __attribute__((always_inline)) {
      return DET && !PART && pd.go && pd.rank > 0;
    };
    // Blocking wait for the turn.
    auto reduce_wait = [&](Pending& pd) __attribute__((always_inline)) {
      if (reduce_needs_turn(pd)) {
        if (cross) {
          // The running sums are then read with device-scope loads, which see the other
          // XCD's device-scope stores without a fence.
          pd.go = wait_turn(pd.sem, pd.rank, p.err, p.timeout_ticks);
        } else {
          pd.go = wait_turn_local(pd.sem, pd.rank, p.err, p.timeout_ticks);
        }
        failed = !pd.go;
        if (failed) pd.acc_rs = make_rsrc(pd.acc_blk, 0);
      }
    };
    // Running sum so far (after the turn has come); the first contributor (and the
    // atomic variant) reads through an empty descriptor, which returns zeros without
    // touching memory.
    auto reduce_load = [&](const Pending& pd, floatx16 (&ld)[C::NBLK]) __attribute__((always_inline)) {
      if (!DET || PART) {
        // The atomic variant adds partials from zero (kZeroStart) and issues no load: a
        // load would make the next wait for it also wait for every float atomic issued
        // before it.
        return;
      }
      const rsrc_t lrs = make_rsrc(pd.acc_blk, reduce_needs_turn(pd) ? 2 * DB * kBlkBytes : 0);
#pragma unroll
      for (int t2 = 0; t2 < C::NBLK; ++t2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // The previous contributor shares this XCD's L2 unless the chains cross XCDs.
          const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(lrs, acc_off[t2] + 1024 * i, 0, cross ? kSC1 : kSC0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned u = v[e];
            ld[t2][4 * i + e] = __builtin_bit_cast(float, u);
          }
        }
      }
    };
    // Stores part i (elements 4 i .. 4 i + 3, i.e. row group t = i) of dQ block t2.
#ifdef DASH_REPLAY
    // Replay builds: the dQ MFMAs start from zero; the running sum loaded for the step
    // is kept here and added to the partial with one fp32 add per element, and every
    // partial is dumped, so that a CPU replay in rank order reproduces the sums bit for bit.
    floatx16 run[C::NBLK];
#endif
    auto reduce_store_part = [&](const Pending& pd, int t2, int i, const floatx16& v_in) __attribute__((always_inline)) {
      if (NODQ) return;
#ifdef DASH_REPLAY
      if (!pd.go) return;
      floatx16 v = v_in;
      if (DET && !PART) {
        if (pd.dump) {
          u32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float f = v_in[4 * i + e];
            x[e] = __builtin_bit_cast(unsigned, f);
          }
          const int blk = w + NW * t2;
          float* dst = pd.dump + static_cast<int64_t>(blk) * p.replay_ranks * kDqBlock + 256 * i + 4 * lane;
          *reinterpret_cast<u32x4*>(dst) = x;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * i + e] = run[t2][4 * i + e] + v_in[4 * i + e];
      }
#else
      const floatx16& v = v_in;
#endif
      if (!DET) {
        // Row-major accumulator; rows past N exist (padding) and are never output. Row
        // of element (t, e), t = i: 32 qb + 16 (t / 2) + 2 (t % 2) + 4 e; the wave-uniform
        // part goes to the scalar offset operand.
        const int qb = (w + NW * t2) / DB;
        const int t = i;
        const int vb = 4 * blk_base(t2);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = v[4 * t + e];
          __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
              x, pd.acc_rs, vb + 16 * (e & 1) * D, 4 * (32 * qb + 16 * (t >> 1) + 2 * (t & 1) + 4 * (e & 2)) * D, 0);
        }
      } else {
        u32x4 x;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // Element copied to a scalar first: a bit-cast of a vector element lvalue
          // reads the vector's first element.
          const float f = v[4 * i + e];
          x[e] = __builtin_bit_cast(unsigned, f);
        }
        // Chains that cross XCDs store with device scope (written through this XCD's L2);
        // inside one XCD the L2 is the coherence point and a plain store suffices.
        __builtin_amdgcn_raw_buffer_store_b128(x, pd.acc_rs, acc_off[t2] + 1024 * i, 0, cross ? kSC1 : 0);
      }
    };
    auto reduce_store = [&](const Pending& pd, int t2, const floatx16& v) __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 4; ++i) reduce_store_part(pd, t2, i, v);
    };
    // Call after wait_mem_done(): this wave's accumulator stores have been acknowledged
    // (in the L2, or past it for device-scope stores), so the turn can be passed on.
    auto reduce_signal = [&](const Pending& pd) __attribute__((always_inline)) {
      if (!DET || PART || !pd.go || pd.last) return;
      if (lane == 0) {
        // Writer and reader share this XCD's L2, where the acknowledged stores already
        // are: a plain store into the L2 suffices, and the next contributor's poll then
        // hits in the L2 instead of going past it. Across XCDs the running sums were
        // stored with device scope, so no L2 write-back is needed before the flag, which
        // is itself a device-scope store.
        __builtin_amdgcn_raw_buffer_store_b32(static_cast<unsigned>(pd.rank + 1), make_rsrc(pd.sem, 4), 0, 0,
                                              cross ? kSC1 : 0);
      }
    };

    // Reduction state carried from step to step: the previous step's contribution, its
    // running sums (or dQ partials once the MFMAs have run) and whether their loads
    // have been issued already.
    // Step 0 has no previous partial: its stores go to a contribution with empty
    // descriptors, which drops them.
    Pending pd;
    pd.rank = 0;
    pd.last = 0;
    pd.sem = p.sem;
    pd.acc_blk = p.dqacc;
    pd.acc_rs = make_rsrc(p.dqacc, 0);
    pd.go = false;
#ifdef DASH_REPLAY
    pd.dump = nullptr;
#endif
    floatx16 ld[C::NBLK];
    bool loaded = false;
    constexpr int kBlkA = (C::NBLK + 1) / 2;  // dQ blocks reduced under the first S/dP block
    for (int s = 0; s < n_steps; ++s) {
      PROF_COUNT(kProfSteps);
      const int buf = (par0 + s) & 1;
      const int q0 = rec_cur.y;
      const int j = q0 / BC;
      const Quad rec_nn = load_quad(steps, t_begin * SUBS + s + 2);  // taken over at the step's end

      // Previous step's reduction: if the poll of the last step found no turn, wait
      // for it here and issue the running-sum loads now.
      const bool have_prev = s > 0;
      if (have_prev && !loaded) {
        PROF_MARK(kProfDq);
        reduce_wait(pd);
        PROF_MARK(kProfWait);
        reduce_load(pd, ld);
        PROF_COUNT(kProfLate);
      }
      PROF_MARK(kProfLoads);

      const LDS_AS char* sQ = smem + C::OFF_Q + buf * C::QT;
      const LDS_AS char* sdO = smem + C::OFF_DO + buf * C::QT;
      const LDS_AS char* sNL = smem + C::OFF_NL + buf * 256;
      const LDS_AS char* sDL = smem + C::OFF_DL + buf * 256;
      LDS_AS char* sdS = smem + C::OFF_DS + buf * C::DST;
      // Only the diagonal task of a causal mask needs a mask: rows past the batch's length
      // have -LSE*log2(e) = -inf (P = 0) and columns past it meet zero K rows in dQ.
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

      // The next step's copies (Q, dO, -LSE*log2e, -D into buffer (s + 1) & 1, free since
      // the last barrier), spread over the S/dP slots: copy op o is Q block o, dO block
      // o - PER_WAVE, then -LSE*log2e (even waves) or -D (odd waves).
      // At the item's last step: the next item's first step. At the worker's last step
      // the next record belongs to another worker (or is a zero record): copied all the
      // same, so that the copies need no branch; nothing reads that buffer any more.
      const int q0_n = rec_nxt.y;
      const int64_t bh_n = rec_nxt.x;
      const int nrow_n = len_of(rec_nxt.x / H);  // rows of the next step's batch
      const bf16* q_n = p.q + bh_n * N * D;
      const bf16* do_n = p.dO + bh_n * N * D;
      LDS_AS char* const sQn = smem + C::OFF_Q + (buf ^ 1) * C::QT;
      LDS_AS char* const sdOn = smem + C::OFF_DO + (buf ^ 1) * C::QT;
      constexpr int kPW = TileCopy<D, BQ, NW>::PER_WAVE;
      constexpr int kCopyOps = 2 * kPW + 1;
      auto copy_op = [&](int o) __attribute__((always_inline)) {
        if (o < kPW) {
          qcopy.issue_one_clamped(sQn, q_n, q0_n, nrow_n, w, o);
        } else if (o < 2 * kPW) {
          qcopy.issue_one_clamped(sdOn, do_n, q0_n, nrow_n, w, o - kPW);
        } else {
          // Row arrays are padded to the tile, so rows q0 .. q0+63 always exist. Waves of
          // one parity write the same values to the same LDS slots.
          const float* row_src = (w & 1) ? p.neg_delta : p.nlse2;
          dma4(row_src + bh_n * p.row_stride + q0_n, row_lane, smem + ((w & 1) ? C::OFF_DL : C::OFF_NL) + (buf ^ 1) * 256);
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
        if (!NODQ && (r0 & 3) == 2) {
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
      // group t + 1 are loaded at the first slot of group t, two slots before they are
      // used (ring of 2), so that their LDS latency is hidden even where the scheduler
      // puts the softmax first in its slot.
      auto softmax_slot = [&](int qb, int slot, const floatx16& S, const floatx16& dP, floatx4 (&nlr)[2],
                              u32x4 (&Pw)[2], u32x4 (&dSw)[2]) __attribute__((always_inline)) {
        const int t = slot >> 1;
        if (!(slot & 1) && t + 1 < 4) nlr[(t + 1) & 1] = load_nl(qb, t + 1);
        softmax2(qb, 2 * slot, S, dP, nlr[t & 1], Pw, dSw);
      };
#define SLOT() __builtin_amdgcn_sched_barrier(0)
      // Operands are read from LDS kPF slots ahead of their MFMAs (rings of kPF + 1).
      constexpr int kPF = 2, kRing = kPF + 1;
      constexpr int NSD = 2 * DK;  // S/dP k-steps of the two 32-row blocks
      constexpr int NIT = 2 * DB;  // dV/dK (hf, db) iterations of one block, 2 MFMAs each
      constexpr int NDV = 2 * NIT;
      static_assert(DK == 8 || DK == 4, "S/dP slots");
      // The previous step's dQ MFMAs (dQ block t2, k-step kk: MFMA number t2 KK + kk) run
      // inside the S/dP slots: blocks [0, kBlkA) under block 0's S/dP, the rest under
      // block 1's, kQ1 / kQ2 of them per slot, their dS operands one slot ahead.
      constexpr int kQ1 = kBlkA * KK / DK, kQ2 = (C::NBLK - kBlkA) * KK / DK;
      static_assert(kQ1 * DK == kBlkA * KK && kQ2 * DK == (C::NBLK - kBlkA) * KK, "dQ MFMAs per slot");
      constexpr int kQmax = kQ1 > kQ2 ? kQ1 : kQ2;
      constexpr int kQRing = 2 * kQmax;
      floatx16 S0, S1;
      floatx16 dP0 = load_negd(0), dP1;
      u32x4 P0[2], dS0[2], P1[2], dS1[2];
      floatx4 nlr[2];
      bf16x8 aq[kRing], ad[kRing], bo[kRing], bq[kRing];
      bf16x8 aqd[kQRing];
      // S/dP k-step i = (block i / DK, k-step i % DK); dV/dK iteration j = (block j / NIT,
      // (hf, db) = j % NIT).
      auto sd_load = [&](int i) __attribute__((always_inline)) {
        aq[i % kRing] = lds_ld16(sQ, sdp_off(i / DK, i % DK));
        ad[i % kRing] = lds_ld16(sdO, sdp_off(i / DK, i % DK));
      };
      auto dv_load = [&](int j) __attribute__((always_inline)) {
        load_bt(j / NIT, j % NIT, bo[j % kRing], bq[j % kRing]);
      };
      // Issued in S/dP slot i: operands kPF slots ahead, across into the dV/dK sequence.
      auto sd_prefetch = [&](int i) __attribute__((always_inline)) {
        if (i + kPF < NSD)
          sd_load(i + kPF);
        else
          dv_load(i + kPF - NSD);
      };
      auto sd_mfma = [&](int i, floatx16& S, floatx16& dP) __attribute__((always_inline)) {
        const int ks = i % DK;
        if (ks == 0)
          mfma32_vab_zero(S, aq[i % kRing], kreg[0]);
        else
          mfma32_vab(S, aq[i % kRing], kreg[ks]);
        mfma32_vab(dP, ad[i % kRing], vreg[ks]);
      };
      // dQ MFMAs of S/dP slot i (previous step's dS^T, LDS buffer buf ^ 1; on an
      // item's first step the MFMAs run on stale data and their results are dropped).
      const LDS_AS char* sdSprev = smem + C::OFF_DS + (buf ^ 1) * C::DST;
      auto dq_first = [&](int i) __attribute__((always_inline)) { return i < DK ? i * kQ1 : kBlkA * KK + (i - DK) * kQ2; };
      auto dq_count = [&](int i) __attribute__((always_inline)) { return i < DK ? kQ1 : kQ2; };
      auto dq_load = [&](int i) __attribute__((always_inline)) {
        if (NODQ) return;
#pragma unroll
        for (int n = 0; n < dq_count(i); ++n) {
          const int m = dq_first(i) + n, t2 = m / KK, kk = m % KK;
          const int off = ds_rd_lane + 16 * kk * kDsStride + 64 * ((w + NW * t2) / DB);
          aqd[m % kQRing] = join(lds_tr(sdSprev, off), lds_tr(sdSprev, off + kDsStride));
        }
      };
      auto dq_mfma = [&](int i) __attribute__((always_inline)) {
        if (NODQ) return;
#pragma unroll
        for (int n = 0; n < dq_count(i); ++n) {
          const int m = dq_first(i) + n, t2 = m / KK, kk = m % KK;
          dq_mma(ld[t2], kk, aqd[m % kQRing], kT[t2 % C::NKD][kk]);
        }
      };
#pragma unroll
      for (int i = 0; i < kPF; ++i) sd_load(i);
      dq_load(0);
      // Every running-sum load has landed before the first copy below is issued: the
      // vector-memory counter is in order, and the compiler, which does not see the
      // copies, would otherwise wait for them too.
#pragma unroll
      for (int t2 = 0; t2 < C::NBLK; ++t2)
        if (!NODQ) asm volatile("" : "+v"(ld[t2]));
      PROF_MARK(kProfItem);
#ifdef DASH_REPLAY
#pragma unroll
      for (int t2 = 0; t2 < C::NBLK; ++t2) run[t2] = ld[t2];
#endif
      SLOT();
      // Block 0: S/dP, with dQ blocks [0, kBlkA) of the previous step and the next
      // step's copies.
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        sd_prefetch(ks);
        if (ks + 1 < NSD) dq_load(ks + 1);
        if (ks == DK / 2) nlr[0] = load_nl(0, 0);
        if (ks == DK / 2) dP1 = load_negd(1);
        sd_mfma(ks, S0, dP0);
        dq_mfma(ks);
#pragma unroll
        for (int o = ks * kCopyOps / DK; o < (ks + 1) * kCopyOps / DK; ++o) copy_op(o);
        SLOT();
      }
      PROF_MARK(kProfSd0);
      mfma_result_wait(S0, dP0);  // before the VALU reads them (and the stores read ld)
#pragma unroll
      for (int t2 = 0; t2 < kBlkA; ++t2)
        if (!NODQ) asm volatile("" : "+v"(ld[t2]));
      if (diag) mask_diag(0, S0);
      PROF_MARK(kProfMid0);
      SLOT();
      // Block 1: S/dP with block 0's softmax (8 slots of 2 elements over the DK k-steps)
      // and the remaining dQ blocks.
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) {
        sd_prefetch(DK + ks);
        if (DK + ks + 1 < NSD) dq_load(DK + ks + 1);
        sd_mfma(DK + ks, S1, dP1);
        dq_mfma(DK + ks);
#pragma unroll
        for (int sl = (8 / DK) * ks; sl < (8 / DK) * (ks + 1); ++sl) softmax_slot(0, sl, S0, dP0, nlr, P0, dS0);
        if (ks == (6 * DK) / 8) nlr[0] = load_nl(1, 0);  // after group 2 of block 0 (slots 4, 5)
        // Stores of the first dQ blocks (4 parts each) over these slots.
#pragma unroll
        for (int x = ks * 4 * kBlkA / DK; x < (ks + 1) * 4 * kBlkA / DK; ++x) reduce_store_part(pd, x / 4, x % 4, ld[x / 4]);
        SLOT();
      }
      PROF_MARK(kProfSd1);
      mfma_result_wait(S1, dP1);
#pragma unroll
      for (int t2 = kBlkA; t2 < C::NBLK; ++t2)
        if (!NODQ) asm volatile("" : "+v"(ld[t2]));
      if (diag) mask_diag(1, S1);
      PROF_MARK(kProfMid1);
      SLOT();
      // The reduction of the current step's partial, prepared during the last phase.
      Pending pd_n;
      int sem_now = 0;
      // dV += P^T dO, dK += dS^T Q over both blocks; block 1's softmax under block 0's.
#pragma unroll
      for (int j = 0; j < NDV; ++j) {
        if (j + kPF < NDV) dv_load(j + kPF);
        const int qb = j / NIT, it = j % NIT;
        const int hf = it / DB, db = it % DB;
        mfma32_acc(accV[db], as_bf16x8(qb ? P1[hf] : P0[hf]), bo[j % kRing]);
        mfma32_acc(accK[db], as_bf16x8(qb ? dS1[hf] : dS0[hf]), bq[j % kRing]);
        if (qb == 0) {
#pragma unroll
          for (int sl = (8 / NIT) * it; sl < (8 / NIT) * (it + 1); ++sl) softmax_slot(1, sl, S1, dP1, nlr, P1, dS1);
          // Stores of the other dQ blocks over the first half of these slots.
          if (2 * it < NIT) {
            constexpr int kB = C::NBLK - kBlkA, kH = NIT / 2;
#pragma unroll
            for (int x = it * 4 * kB / kH; x < (it + 1) * 4 * kB / kH; ++x)
              reduce_store_part(pd, kBlkA + x / 4, x % 4, ld[kBlkA + x / 4]);
          }
        }
        if (j + 1 == NIT) {
          PROF_MARK(kProfDv0);
          // Stores and copies acknowledged (the copies were issued a phase earlier):
          // the turn is passed on; the next step's tiles are in LDS. The atomic variant
          // passes no turn: it waits for the copies only, and its float atomics, all
          // issued after the copies, stay in flight (the vector-memory counter drains in
          // issue order).
          if (DET) {
            wait_mem_done();
          } else {
            constexpr int kAtomics = NODQ ? 0 : (16 * C::NBLK < 63 ? 16 * C::NBLK : 63);
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __builtin_amdgcn_s_waitcnt(wait_vmcnt(kAtomics));
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
          }
          if (have_prev) reduce_signal(pd);
          PROF_MARK(kProfReduce);
        }
        if (j == NIT) {
          // This step's contribution: bookkeeping and a poll of its turn (a plain load,
          // not waited for until half a phase later).
          // The load is issued and its value read on every step (through an empty
          // descriptor, which returns 0, when no turn is needed): a load into a register
          // that some path leaves unread makes the compiler wait for all vector memory
          // (the running-sum loads included) before the register is reused.
          pd_n = reduce_prepare(rec_cur);
          if (DET) {
            const rsrc_t srs = make_rsrc(pd_n.sem, reduce_needs_turn(pd_n) ? 4 : 0);
            sem_now = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(srs, 0, 0, cross ? kSC1 : kSC0));
          }
        }
        if (j == NIT + NIT / 2) {
          PROF_MARK(kProfBody);
          const int sem_seen = __builtin_amdgcn_readfirstlane(sem_now);
          loaded = !reduce_needs_turn(pd_n) || sem_seen == pd_n.rank;
          PROF_MARK(kProfPoll);
          if (loaded) reduce_load(pd_n, ld);  // (device-scope loads across XCDs: no fence)
        }
        SLOT();
      }
#undef SLOT
      pd = pd_n;
      PROF_MARK(kProfBody);
      // dS^T of all waves is visible after the barrier (the copies were awaited above;
      // the running-sum loads stay in flight across it). The wait is the compiler's own
      // s_waitcnt, so that it also counts as the wait for the step record read ahead.
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      rec_cur = rec_nxt;
      rec_nxt = rec_nn;
      // The step's dV/dK MFMAs are done: wait for them before anything else can read the
      // accumulators. On every step, at the end of the loop body, so that the wait also
      // precedes the copies of the accumulators the compiler may place on the loop's exit
      // edge (and reads in the epilogue).
      mfma_settle(accK, accV);
      PROF_MARK(kProfBarrier);
    }
    // The item's last step: its dQ partial and reduction.
    {
      if (!loaded) {
        reduce_wait(pd);
        reduce_load(pd, ld);
      }
#pragma unroll
      for (int t2 = 0; t2 < C::NBLK; ++t2) {
#ifdef DASH_REPLAY
        run[t2] = ld[t2];
#endif
        dq_block(n_steps - 1, t2, ld[t2]);
        reduce_store(pd, t2, ld[t2]);
      }
      PROF_MARK(kProfFlush);
      wait_mem_done();
      reduce_signal(pd);
      PROF_MARK(kProfReduce);
    }
    // The next item's K and V tiles (the last step's barrier has passed: no wave reads
    // the K tile or the last step's buffer any more). Its step 0 uses the buffer the last
    // step's copies went to.
    par0 = (par0 + n_steps) & 1;
    if (has_next) issue_kv(it + 1, par0);

    // Epilogue: dK = s dK, dV; bf16 stores of this wave's 32 KV rows. A lane holds one
    // column of each 32x32 block, so the rows are put together in LDS first: in this
    // wave's 32 rows of the dS^T buffer that the next item's step 0 writes (free since the
    // last step's barrier, and the next item's prologue barrier comes before that step),
    // 64 columns at a time; then every lane stores 16-byte row chunks.
    LDS_AS char* stage = smem + C::OFF_DS + par0 * C::DST + 32 * w * kDsStride;
    bf16* dKg = p.dk + bg * N * D;
    bf16* dVg = p.dv + bg * N * D;
#pragma unroll
    for (int tns = 0; tns < 2; ++tns) {
      const floatx16* acc = tns == 0 ? accK : accV;
      const float mul = tns == 0 ? p.scale : 1.f;
      bf16* g = tns == 0 ? dKg : dVg;
#pragma unroll
      for (int half = 0; half < DB / 2; ++half) {
        // Element r of block 2 half + e2: row 8 (r / 4) + 4 hi + r % 4, column 32 e2 + l32.
#pragma unroll
        for (int e2 = 0; e2 < 2; ++e2)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * hi + (r & 3);
            *reinterpret_cast<LDS_AS bf16*>(stage + row * kDsStride + 2 * (32 * e2 + l32)) =
                static_cast<bf16>(acc[2 * half + e2][r] * mul);
          }
        // 32 rows x 128 bytes: chunk lane + 64 k is 16 bytes of row chunk / 8.
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int chunk = lane + 64 * k, row = chunk >> 3, c16 = chunk & 7;
          const u32x4 v = *reinterpret_cast<const LDS_AS u32x4*>(stage + row * kDsStride + 16 * c16);
          const int kvr = kv0 + 32 * w + row;
          if (kvr < nrow) *reinterpret_cast<u32x4*>(g + static_cast<int64_t>(kvr) * D + 64 * half + 8 * c16) = v;
        }
      }
    }
    // (No barrier here: the next item's prologue waits for its tiles and synchronises.)
    PROF_MARK(kProfEpi);
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
  auto fn = prm.deterministic == 2 ? bwd_main_kernel<D, NW, false, false, true, false>
            : prm.deterministic == 3 ? bwd_main_kernel<D, NW, true, false, false, true>
            : !prm.deterministic     ? bwd_main_kernel<D, NW, false, false, false, false>
            : prm.xcd_local          ? bwd_main_kernel<D, NW, true, false, false, false>
                                     : bwd_main_kernel<D, NW, true, true, false, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, shmem);
  if (e != hipSuccess) return e;
  BwdParams local = prm;
  void* args[] = {&local};
  return launch_resident(reinterpret_cast<const void*>(fn), grid, NW * 64, shmem, args, stream);
}

// One (d, waves) instantiation per translation unit, selected by DASH_MAIN_D and
// DASH_MAIN_NW, so that each can get its own code-generation flags.
#define DASH_CAT2(a, b, c, d) a##b##c##d
#define DASH_CAT(a, b, c, d) DASH_CAT2(a, b, c, d)
hipError_t DASH_CAT(launch_main_d, DASH_MAIN_D, _nw, DASH_MAIN_NW)(const BwdParams& prm, int grid, hipStream_t stream) {
  return launch_main_t<DASH_MAIN_D, DASH_MAIN_NW>(prm, grid, stream);
}

}  // namespace dash
