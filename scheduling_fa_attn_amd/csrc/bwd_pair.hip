// Main HIP kernel of the deterministic attention backward for gfx950 (MI355X), two
// waves per SIMD (head dimension 128 or 64, 128-row tiles).
//
// Math (DASH paper, arXiv 2601.21824, section 2.1; "Writing an Attention Kernel",
// section "In the real world"): per (batch b, query head h, key/value head g):
//   P  = exp(s Q K^T - LSE)   (recomputed, masked entries 0)
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D)
//   dK = s dS^T Q,  dQ = s dS K
// Work decomposition (DASH paper, section 2.1, Fig. 1 left; section 3.1): a workgroup
// owns one 128-row KV tile at a time and keeps its dK/dV in registers while it visits
// the Q tiles the schedule table lists; the dQ partial of every visit is added to an
// fp32 accumulator in global memory in the order the table fixes (ordered reduction),
// or with float atomics (the non-deterministic variant kept for comparison).
//
// Why a second kernel. A wave that owns 32 KV rows and does all five contractions needs
// about 450 registers at d = 128 (dK and dV accumulators, K and V operands, K^T for the
// dQ contraction, plus the S/dP accumulators and operands in flight), so only one wave
// fits per SIMD and that wave alone must hide every LDS, memory and VALU latency. Here
// the same 32 KV rows are shared by a pair of waves that split the work by role:
//   wave A (waves 0-3, pair p = w):     S = Q K^T, P = exp2(...), dV += P^T dO
//   wave B (waves 4-7, pair p = w - 4): dP - D = dO V^T - D, dS = P (dP - D), dK += dS^T Q
// and each wave computes one 32x32 block of the step's 64 x 128 dQ partial (dS K). Per
// wave and 64-row step that is 40 MFMAs (16 + 16 + 8) and about 250 registers: a K or V
// operand (32 AGPRs), K^T of one d block (32), one accumulator (dV or dK, 64) and the
// VGPRs in flight, so the two waves of a pair share one SIMD and each covers the other's
// stalls. At d = 64 the step's partial has four 32x32 blocks: the A waves compute them
// (24 MFMAs per A wave and step, 16 per B wave). P goes from A to B as bf16 through a
// 4 KiB LDS area per pair (lane l of B holds the same S/dP accumulator elements as lane
// l of A); dS goes to LDS transposed, as the dQ contraction needs it anyway.
//
// Step of 64 Q rows (a pair-local handoff X and a workgroup barrier Y):
//   A: S MFMAs of Q block 0 with the next step's Q-tile copies between them, then of
//      block 1 with block 0's softmax between them; block 1's softmax; P -> LDS
//                                                                   | flag X set |
//      dV MFMAs with the previous step's dQ MFMAs between those of the first half (one
//      per dV MFMA at d = 128, two at d = 64), their stores (acknowledged under the second
//      half), the turn passed on; this step's turn polled and running sum loaded
//                                                                   | barrier Y |
//   B: dP MFMAs with the next step's dO-tile copies and the previous step's dQ block;
//      its stores                                                   | flag X awaited |
//      P from LDS; dS of block 0 (registers, and transposed to LDS); dK MFMAs of
//      block 0 with block 1's dS between them; dK MFMAs of block 1; the previous step's
//      turn passed on; this step's turn polled and running sum loaded | barrier Y |
// X synchronises only the two waves of a pair (an LDS flag holding the number of the
// step whose P is in the pair's exchange area; A writes it after its P stores have
// completed, B polls it), so that pairs do not wait for each other mid-step; Y is the
// workgroup barrier that publishes every pair's dS^T and the next step's tiles.
// At d = 128 the A waves copy the next step's Q tile (during their first S MFMAs, as early
// as the step allows: the buffer was last read in the step before) and the B waves its dO
// tile (during their dP MFMAs); at d = 64, where the A waves own every dQ block
// and the B waves have slack before the P handoff, the B waves copy both. The compiler
// does not see these copies (inline assembly), so a wave waits for its running-sum loads
// before issuing them (the vector-memory counter is in order) and for the copies
// themselves before the step-end barrier.
// Variable-length batches: every row limit (copy clamps, the zeroed K rows of a ragged
// KV tile, the dK/dV stores) is the length of the item's or step's batch; N stays the
// row stride.
// Operand layouts, the padded and row-permuted LDS tiles, the fp32 accumulator's block
// layout, the step records and the turn protocol are those of bwd_main.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernels.h"

// Depth of the LDS operand rings (reads issued DASH_PAIR_RING - 1 MFMAs ahead). Depths
// 3 and 4 measured no faster than 2 (two waves per SIMD cover the LDS latency that a
// deeper ring would) and spill a few registers.
#ifndef DASH_PAIR_RING
#define DASH_PAIR_RING 2
#endif

namespace dash {

template <int D>
struct PairCfg {
  static constexpr int NW = 8;          // waves: four pairs
  static constexpr int NP = 4;          // pairs (KV row blocks of 32)
  static constexpr int BC = 128;        // KV (and Q) tile rows
  static constexpr int BQ = 64;         // Q rows per step
  static constexpr int SUBS = BC / BQ;  // steps per task
  static constexpr int NT = NW * 64;
  static constexpr int DB = D / 32;     // 32-column blocks of d
  static constexpr int DK = D / 16;     // k-steps over d
  static constexpr int KK = BC / 16;    // k-steps over the KV tile
  static constexpr int ST = TileGeom<D>::STRIDE;
  static constexpr int QT = BQ * ST;
  static constexpr int DST = BC * kDsStride;
  static constexpr int PXW = 4096;      // P exchange per pair: 4 x 16 bytes per lane
  static constexpr int OFF_Q = 0;                 // 2 buffers
  static constexpr int OFF_DO = OFF_Q + 2 * QT;   // 2 buffers
  static constexpr int OFF_DS = OFF_DO + 2 * QT;  // 2 buffers
  static constexpr int OFF_K = OFF_DS + 2 * DST;  // K tile [BC][D]
  static constexpr int OFF_PX = OFF_K + BC * ST;  // P exchange, NP x PXW
  static constexpr int OFF_NL = OFF_PX + NP * PXW;  // 2 x 64 floats: -LSE*log2(e)
  static constexpr int OFF_DL = OFF_NL + 2 * 256;   // 2 x 64 floats: -D
  static constexpr int OFF_MISC = OFF_DL + 2 * 256;
  static constexpr int BYTES = OFF_MISC + 64;
  // dQ blocks of a step's 64 x D partial: one per wave at D = 128; at D = 64 the four
  // blocks go to the A waves and the B waves compute no dQ.
  static_assert(2 * DB == NW || 2 * DB == NW / 2, "one 32x32 dQ block per wave, or per A wave");
  static constexpr bool kAllWavesDq = 2 * DB == NW;
  static_assert(BYTES <= 160 * 1024, "LDS of one CU");
  static_assert(QT % 1024 == 0 && DST % 1024 == 0 && (BC * ST) % 1024 == 0, "1 KiB-aligned tiles");
};

// The value of lane l ^ B (B = 1, 2, 4: inside the lane's group of 8) by data-parallel
// primitives (no LDS): quad permutations for 1 and 2; for 4, a row shift by 4 in the
// direction that stays inside the group (row_shl: lane l reads lane l + 4).
template <int B>
__device__ __forceinline__ unsigned lane_xor(unsigned x, int ln) {
  const int v = static_cast<int>(x);
  if constexpr (B == 1) {
    return static_cast<unsigned>(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  } else if constexpr (B == 2) {
    return static_cast<unsigned>(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  } else {
    static_assert(B == 4, "lane distance 1, 2 or 4");
    const int from_hi = __builtin_amdgcn_mov_dpp(v, 0x104, 0xF, 0xF, false);  // row_shl:4
    const int from_lo = __builtin_amdgcn_mov_dpp(v, 0x114, 0xF, 0xF, false);  // row_shr:4
    return static_cast<unsigned>((ln & 4) ? from_lo : from_hi);
  }
}

// One round of the 8 x 8 transpose of u32 across 8 lanes (lane distance B): lanes with
// bit B set send their slot m and take the partner's slot m ^ B into slot m; the others
// send slot m ^ B and take the partner's slot m into it (m with bit B clear). The selects
// are written with a mask: as a ? b : c on the array elements the compiler turns them
// into dynamic indexing over all eight slots.
template <int B>
__device__ __forceinline__ void xchg_stage(unsigned (&P)[8], int ln) {
  const unsigned up = 0u - ((static_cast<unsigned>(ln) / B) & 1u);
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    if (m & B) continue;
    const unsigned lo_m = P[m], hi_m = P[m ^ B];
    const unsigned x = hi_m ^ ((lo_m ^ hi_m) & up);
    const unsigned y = lane_xor<B>(x, ln);
    P[m] = lo_m ^ ((lo_m ^ y) & up);
    P[m ^ B] = y ^ ((y ^ hi_m) & up);
  }
}

// (B's dQ MFMAs, at D = 128, run in the last KK slots of its 2 DK dP slots, with their
// operands prefetched from the slot before.)
// Body of the kernel for one role (ROLE_A: waves 0-3, else waves 4-7). Each role is
// its own inlined copy, so that the register allocator never sees the values of one
// role live in the other's code.
template <int D, bool DET, bool ROLE_A, bool PART, bool FUSED>
__device__ __forceinline__ void pair_body(const BwdParams& p, LDS_AS char* smem, int worker, int w) {
  using C = PairCfg<D>;
  constexpr int BC = C::BC, BQ = C::BQ, SUBS = C::SUBS, DB = C::DB, DK = C::DK, KK = C::KK, ST = C::ST;
  constexpr bool roleA = ROLE_A;
  // This wave's dQ block (32 Q rows x 32 d columns of the step's partial) and whether it
  // has one: block dqb is Q block dqb / DB, d block dqb % DB.
  constexpr bool HAS_DQ = C::kAllWavesDq || ROLE_A;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int pr = w & 3;  // pair: KV rows 32 pr .. 32 pr + 31 of the tile
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int L16 = lane & 15;
  const int nb = (lane >> 4) & 1;
  PROF_DECL
  const int H = p.H, Hkv = p.Hkv, N = p.N;
  // Rows of batch b: N, or seqlens[b] <= N for variable-length batches (N stays the row
  // stride of every tensor; rows past a batch's length are padding, never read as data).
  const CONST_AS int* seqlens = (const CONST_AS int*)p.seqlens;
  auto len_of = [&](int b) __attribute__((always_inline)) { return p.seqlens ? seqlens[b] : N; };
  bool failed = false;  // this wave gave up waiting (error reported); it keeps going without reducing
  const CONST_AS int* worker_begin = (const CONST_AS int*)p.worker_begin;
  const CONST_AS Quad* items = (const CONST_AS Quad*)p.items;
  const CONST_AS Quad* tasks = (const CONST_AS Quad*)p.tasks;
  const int it_begin = worker_begin[worker];
  const int it_end = worker_begin[worker + 1];

  // Per-lane parts of the LDS addresses (as in bwd_main.hip).
  const int a_lane = pi16(l32) * ST + 16 * hi;
  const int bt_lane = (hi + 4 * (L16 >> 2)) * ST + 2 * (16 * nb + 4 * (L16 & 3));
  const int kvrow_lane = 2 * hi + 4 * (L16 >> 2);
  const int col_lane2 = 2 * (16 * nb + 4 * (L16 & 3));
  const int ds_rd_lane = kvrow_lane * kDsStride + col_lane2;
  const int kd_lane = kvrow_lane * ST + col_lane2;
  const int ds_wr_lane = (32 * pr + l32) * kDsStride + 8 * hi;
  LDS_AS char* const sK = smem + C::OFF_K;
  LDS_AS char* const sPX = smem + C::OFF_PX + pr * C::PXW + 16 * lane;  // + 1024 c
  // The pair's P-ready flag: the number of the step whose P is in the exchange area.
  volatile LDS_AS int* const sFlag = reinterpret_cast<volatile LDS_AS int*>(smem + C::OFF_MISC + 16) + pr;
  int gstep = 0;  // steps begun by this wave (the same sequence in both waves of a pair)

  // Copies are issued by the four B waves (wave index pr in the copy plans). The plans
  // are built where they are used, from the lane index passed through an empty asm, so
  // that their per-lane offsets are not hoisted out of the loops and kept live.
  auto opaque_lane = [&]() __attribute__((always_inline)) {
    int l = lane;
    asm volatile("" : "+v"(l));
    return l;
  };
  const unsigned row_lane = static_cast<unsigned>(pi16(lane) * 4);  // LDS slot m <- row pi(m)

  // An item's tiles, copied while the previous item finishes (B waves): K -> the K tile;
  // V -> the Q and dO areas of the buffer its step 0 does not use; the first step's Q,
  // dO, -LSE*log2e, -D -> the buffer of its step 0.
  auto issue_kv = [&](int it2, int par0) __attribute__((always_inline)) {
    const Quad item2 = load_quad(items, it2);
    const int64_t bg2 = static_cast<int64_t>(item2.x) * Hkv + item2.y;
    const int kv02 = item2.z * BC;
    const int nb2 = len_of(item2.x);
    TileCopy<D, BC, 4> kcopy;
    kcopy.init(pr, opaque_lane());
    kcopy.issue(sK, p.k + bg2 * N * D, kv02, nb2, pr);
    TileCopy<D, BQ, 4> qcopy;
    qcopy.init(pr, opaque_lane());
#pragma unroll
    for (int hh = 0; hh < BC / BQ; ++hh)
      qcopy.issue(smem + (hh == 0 ? C::OFF_Q : C::OFF_DO) + (par0 ^ 1) * C::QT, p.v + bg2 * N * D, kv02 + BQ * hh,
                  nb2, pr);
  };
  auto issue_first_step = [&](int it2, int par0) __attribute__((always_inline)) {
    const Quad item2 = load_quad(items, it2);
    const Quad task = load_quad(tasks, item2.w);
    const int q0 = task.y * BC;
    const int64_t bh = static_cast<int64_t>(item2.x) * H + task.x;
    const int nb2 = len_of(item2.x);
    TileCopy<D, BQ, 4> qcopy;
    qcopy.init(pr, opaque_lane());
    qcopy.issue(smem + C::OFF_Q + par0 * C::QT, p.q + bh * N * D, q0, nb2, pr);
    qcopy.issue(smem + C::OFF_DO + par0 * C::QT, p.dO + bh * N * D, q0, nb2, pr);
    if (pr == 0) dma4(p.nlse2 + bh * p.row_stride + q0, row_lane, smem + C::OFF_NL + par0 * 256);
    if (pr == 1) dma4(p.neg_delta + bh * p.row_stride + q0, row_lane, smem + C::OFF_DL + par0 * 256);
  };
  int par0 = 0;  // buffer of the current item's step 0
  // Step records {b * H + h, first Q row, rank, last}, read two steps ahead.
  const CONST_AS Quad* steps = (const CONST_AS Quad*)p.steps;
  Quad rec_cur = {0, 0, 0, 0}, rec_nxt = {0, 0, 0, 0};
  if (it_begin < it_end) {
    if (!roleA) {
      issue_kv(it_begin, par0);
      issue_first_step(it_begin, par0);
    }
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
    const int nb = len_of(item.x);  // rows of this item's batch
    const bool has_next = it + 1 < it_end;

    // Item prologue: the item's tiles have landed; the K (A) or V (B) rows of the pair
    // and K^T of this wave's dQ d block to AGPRs; accumulator zeroed.
    wait_mem_done();
    __syncthreads();
    if (kv0 + BC > nb) {
      // Ragged KV tile: K rows past the batch's length become zero, so that dS of those
      // columns adds nothing to dQ; their dK/dV rows are never stored.
      const int r0 = nb - kv0;
      LDS_AS floatx4* z = reinterpret_cast<LDS_AS floatx4*>(sK + r0 * ST);
      int x0 = tid;
      asm volatile("" : "+v"(x0));  // (computed here, not kept live from the kernel's start)
      for (int x = x0; x < (BC - r0) * ST / 16; x += C::NT) z[x] = floatx4{0.f, 0.f, 0.f, 0.f};
      __syncthreads();
    }
    bf16x8 kv[DK];  // A: K rows (B operand of S), B: V rows (B operand of dP)
    {
      const int r = 32 * pr + l32;
      const LDS_AS char* row = roleA ? sK + r * ST
                                     : smem + (r < BQ ? C::OFF_Q : C::OFF_DO) + (par0 ^ 1) * C::QT + (r % BQ) * ST;
#pragma unroll
      for (int ks = 0; ks < DK; ++ks) kv[ks] = to_agpr(lds_ld16(row, 32 * ks + 16 * hi));
    }
    floatx16 acc[DB];  // A: dV, B: dK (unscaled) of the pair's 32 KV rows
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = floatx16{};
    const int kvcol = kv0 + 32 * pr + l32;  // this lane's KV row in S, P, dP, dS
    // dQ block of this wave: Q rows 32 (w / 4) .. of the step, d columns 32 pr ..; its B
    // operand K^T (k-step kk: KV rows 16 kk .. 16 kk + 15 in the dS operand's order).
    const int dqb = C::kAllWavesDq ? w : pr;
    const int qbq = dqb / DB, dbq = dqb % DB;
    bf16x8 kT[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int koff = kd_lane + 16 * kk * ST + 64 * dbq;
      kT[kk] = HAS_DQ ? to_agpr(join(lds_tr(sK, koff), lds_tr(sK, koff + ST))) : bf16x8{};
    }
    __syncthreads();
    PROF_MARK(kProfPro);

#ifdef DASH_REPLAY
    constexpr bool kZeroStart = true;
#else
    constexpr bool kZeroStart = !DET || PART;
#endif
    auto dq_mma = [&](floatx16& a, int kk, const bf16x8& x, const bf16x8& y) __attribute__((always_inline)) {
      if (kZeroStart && kk == 0)
        mfma32_vab_zero(a, x, y);
      else
        mfma32_vab(a, x, y);
    };
    // A operand of dQ k-step kk: dS (transpose reads of dS^T in buffer `sds`).
    auto dq_opnd = [&](const LDS_AS char* sds, int kk) __attribute__((always_inline)) -> bf16x8 {
      const int off = ds_rd_lane + 16 * kk * kDsStride + 64 * qbq;
      return join(lds_tr(sds, off), lds_tr(sds, off + kDsStride));
    };

    constexpr int kBlkBytes = kDqBlock * 4;
    // Ordered variant: this lane's first 4 floats in block w of the step's 2 DB blocks.
    const int acc_off = lane * 16 + dqb * kBlkBytes;
    struct Pending {
      int rank, last;
      int* sem;
      float* acc_blk;  // the step's first fp32 accumulator block
      rsrc_t acc_rs;   // stores (atomic variant: rows q0 .. q0 + 63, row-major); empty if none
      int bhq[FUSED ? 2 : 0];  // FUSED: the step's b * H + h and first Q row (the bf16 dQ rows)
      bool go;
#ifdef DASH_REPLAY
      float* dump;
#endif
    };
    auto reduce_prepare = [&](const Quad& rec) __attribute__((always_inline)) -> Pending {
      Pending pd;
      pd.rank = rec.z;
      pd.last = rec.w;
      const int q0s = rec.y;
      const int64_t bh = rec.x;
      if constexpr (FUSED) {
        pd.bhq[0] = rec.x;
        pd.bhq[1] = rec.y;
      }
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
      pd.sem = p.sem + bh * p.sem_stride + (q0s / BQ) * kSemPerStep + dqb;
#ifdef DASH_REPLAY
      pd.dump = p.replay ? p.replay + (((bh * (p.row_stride / BQ) + q0s / BQ) * (2 * DB)) * p.replay_ranks + pd.rank) *
                                          static_cast<int64_t>(kDqBlock)
                         : nullptr;
#endif
      return pd;
    };
    auto reduce_needs_turn = [&](const Pending& pd) __attribute__((always_inline)) {
      return HAS_DQ && DET && !PART && pd.go && pd.rank > 0;
    };
    auto reduce_wait = [&](Pending& pd) __attribute__((always_inline)) {
      if (reduce_needs_turn(pd)) {
        pd.go = wait_turn_local(pd.sem, pd.rank, p.err, p.timeout_ticks);
        failed = !pd.go;
        if (failed) pd.acc_rs = make_rsrc(pd.acc_blk, 0);
      }
    };
    // Running sum so far; the first contributor reads through an empty descriptor (zeros).
    auto reduce_load = [&](const Pending& pd, floatx16& ld) __attribute__((always_inline)) {
      if (!DET || PART || !HAS_DQ) return;
      const rsrc_t lrs = make_rsrc(pd.acc_blk, reduce_needs_turn(pd) ? 2 * DB * kBlkBytes : 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(lrs, acc_off, 1024 * i, kSC0);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned u = v[e];
          ld[4 * i + e] = __builtin_bit_cast(float, u);
        }
      }
    };
#ifdef DASH_REPLAY
    floatx16 run;  // replay builds: running sum loaded for the partial being reduced
#endif
    // The final sum of this wave's 32x32 dQ block as bf16 rows of dq. Element 4 i + e of
    // lane l is row 16 (i / 2) + 2 (i % 2) + l / 32 + 4 e, column l % 32 of the block, so
    // each group of 8 lanes holds 8 adjacent columns of the same 16 rows: elements 0-7
    // (rows R(m) = 2 (m / 4) + 4 (m % 4) + l / 32) and 8-15 (rows 16 + R(m)) are packed
    // in pairs (one u32 per m), the 8 x 8 block of u32 is transposed across the 8 lanes
    // (three exchange rounds, lane distances 4, 2, 1), and lane k of the group then holds
    // rows R(k) and 16 + R(k), 8 columns each: two 16-byte stores. Rows at or past the
    // batch's length fall outside the descriptor and are dropped.
    auto store_dq_final = [&](const Pending& pd, const floatx16& v) __attribute__((always_inline)) {
      // (Lane-derived values from an opaque lane index, so that the compiler computes them
      // here instead of keeping them live from the kernel's start.)
      const int ln = opaque_lane();
      unsigned P[8];
#pragma unroll
      for (int m = 0; m < 8; ++m) P[m] = pack_bf16(v[m] * p.scale, v[8 + m] * p.scale);
      xchg_stage<4>(P, ln);
      xchg_stage<2>(P, ln);
      xchg_stage<1>(P, ln);
      u32x4 lo, hi4;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        lo[t] = __builtin_amdgcn_perm(P[2 * t + 1], P[2 * t], 0x05040100u);
        hi4[t] = __builtin_amdgcn_perm(P[2 * t + 1], P[2 * t], 0x07060302u);
      }
      // A failed wait leaves the descriptor empty; a step of a ragged last tile may start
      // at or past the length (no rows then).
      const int bh = pd.bhq[0], q0s = pd.bhq[1];
      const int nrow = (p.seqlens ? seqlens[bh / H] : N) - q0s;
      const int rows = !pd.go || nrow <= 0 ? 0 : (nrow < 64 ? nrow : 64);
      const rsrc_t rs = make_rsrc(p.dq + (static_cast<int64_t>(bh) * N + q0s) * D, rows * D * 2);
      const int k = ln & 7;
      const int row = 32 * qbq + 2 * (k >> 2) + 4 * (k & 3) + (ln >> 5);
      const int off = (row * D + 32 * dbq + 8 * ((ln & 31) >> 3)) * 2;
      __builtin_amdgcn_raw_buffer_store_b128(lo, rs, off, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(hi4, rs, off + 16 * D * 2, 0, 0);
    };
    // Whether this step's contribution is the last of its dQ block and goes to dq as bf16
    // (FUSED). The flag goes through an empty asm: otherwise the compiler sees the same
    // test again in reduce_signal and duplicates the code between the two for each
    // outcome.
    auto writes_dq = [&](const Pending& pd) __attribute__((always_inline)) {
      if constexpr (!(FUSED && DET && !PART && HAS_DQ)) {
        return false;
      } else {
        int last = __builtin_amdgcn_readfirstlane(pd.last);
        asm volatile("" : "+s"(last));
        return last != 0;
      }
    };
    auto reduce_store = [&](const Pending& pd, const floatx16& v_in) __attribute__((always_inline)) {
      if (!HAS_DQ) return;
#ifdef DASH_REPLAY
      if (!pd.go) return;
      floatx16 v = v_in;
      if (DET && !PART) {
        if (pd.dump) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            u32x4 x;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float f = v_in[4 * i + e];
              x[e] = __builtin_bit_cast(unsigned, f);
            }
            float* dst = pd.dump + static_cast<int64_t>(dqb) * p.replay_ranks * kDqBlock + 256 * i + 4 * lane;
            *reinterpret_cast<u32x4*>(dst) = x;
          }
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = run[e] + v_in[e];
      }
#else
      const floatx16& v = v_in;
#endif
      if (writes_dq(pd)) {
        store_dq_final(pd, v);
#ifndef DASH_REPLAY
        return;  // (replay builds also keep the final fp32 sum for the exact check)
#endif
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!DET) {
          // Row-major accumulator; element (t = i, e) sits at row 32 qbq + 16 (t / 2) +
          // 2 (t % 2) + hi + 4 e, column 32 dbq + l32.
          const int t = i;
          const int vb = 4 * (hi * D + 32 * dbq + l32);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = v[4 * t + e];
            __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(
                x, pd.acc_rs, vb + 16 * (e & 1) * D, 4 * (32 * qbq + 16 * (t >> 1) + 2 * (t & 1) + 4 * (e & 2)) * D, 0);
          }
        } else {
          u32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float f = v[4 * i + e];
            x[e] = __builtin_bit_cast(unsigned, f);
          }
          __builtin_amdgcn_raw_buffer_store_b128(x, pd.acc_rs, acc_off, 1024 * i, 0);
        }
      }
    };
    // After wait_mem_done(): this wave's accumulator stores are in the L2.
    auto reduce_signal = [&](const Pending& pd) __attribute__((always_inline)) {
      if (!HAS_DQ || !DET || PART || !pd.go || pd.last) return;
      if (lane == 0)
        __builtin_amdgcn_raw_buffer_store_b32(static_cast<unsigned>(pd.rank + 1), make_rsrc(pd.sem, 4), 0, 0, 0);
    };
    // Poll of the turn: a plain load whose value is read later (issued on every step,
    // through an empty descriptor when no turn is needed).
    auto reduce_poll = [&](const Pending& pd) __attribute__((always_inline)) -> int {
      if (!DET || PART || !HAS_DQ) return 0;
      const rsrc_t srs = make_rsrc(pd.sem, reduce_needs_turn(pd) ? 4 : 0);
      return static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(srs, 0, 0, kSC0));
    };

    Pending pd;
    pd.rank = 0;
    pd.last = 0;
    pd.sem = p.sem;
    pd.acc_blk = p.dqacc;
    pd.acc_rs = make_rsrc(p.dqacc, 0);
    if constexpr (FUSED) {
      pd.bhq[0] = 0;
      pd.bhq[1] = 0;
    }
    pd.go = false;
#ifdef DASH_REPLAY
    pd.dump = nullptr;
#endif
    floatx16 ld = {};
    bool loaded = false;
    for (int s = 0; s < n_steps; ++s) {
      PROF_COUNT(kProfSteps);
      ++gstep;
      const int buf = (par0 + s) & 1;
      const int q0 = rec_cur.y;
      const int j = q0 / BC;
      const Quad rec_nn = load_quad(steps, t_begin * SUBS + s + 2);
      const bool have_prev = s > 0;
      const LDS_AS char* sQ = smem + C::OFF_Q + buf * C::QT;
      const LDS_AS char* sdO = smem + C::OFF_DO + buf * C::QT;
      const LDS_AS char* sNL = smem + C::OFF_NL + buf * 256;
      const LDS_AS char* sDL = smem + C::OFF_DL + buf * 256;
      LDS_AS char* sdS = smem + C::OFF_DS + buf * C::DST;
      const LDS_AS char* sdSprev = smem + C::OFF_DS + (buf ^ 1) * C::DST;
      // S, dP A operands (Q or dO rows), block qb, k-step ks.
      auto sdp_off = [&](int qb, int ks) __attribute__((always_inline)) { return a_lane + 32 * qb * ST + 32 * ks; };
      // dV / dK B operands (transpose reads of dO or Q), iteration jj = (qb, hf, db).
      constexpr int NIT = 2 * DB;
      auto bt_load = [&](const LDS_AS char* tile, int jj) __attribute__((always_inline)) -> bf16x8 {
        const int qb = jj / NIT, itr = jj % NIT;
        const int off = bt_lane + (32 * qb + 16 * (itr / DB)) * ST + 64 * (itr % DB);
        return join(lds_tr(tile, off), lds_tr(tile, off + 2 * ST));
      };
#define SLOT() __builtin_amdgcn_sched_barrier(0)
      // Operand rings: LDS reads issued kR - 1 slots ahead of their MFMAs.
      constexpr int kR = DASH_PAIR_RING;
      // The next step's tiles, into buffer buf ^ 1 (free since the last barrier): A waves
      // copy the Q tile and -LSE*log2e, B waves the dO tile and -D. Copy op o < kPW is
      // block pr + 4 o of the tile: LDS slot 64 blk + lane holds chunk c of row r (pad
      // slots re-read chunk 0); rows past N repeat row N - 1. The lane's offset is
      // recomputed at every step rather than kept in a register. At an item's last step
      // the next record is the next item's first step; at the worker's last step it is
      // another worker's (or a zero) record, copied all the same: nothing reads it.
      constexpr int kPW = TileCopy<D, BQ, 4>::PER_WAVE;
      constexpr int kQNI = TileCopy<D, BQ, 4>::NI;
      constexpr int kCopyOps = kPW + 1;
      const int q0_n = rec_nxt.y;
      const int64_t bh_n = rec_nxt.x;
      const int nb_n = p.seqlens ? seqlens[rec_nxt.x / H] : N;  // rows of the next step's batch
      // At d = 64 the B waves copy both tiles (A's running sums then need not land
      // before its S phase's copies, as the copies are invisible to the compiler).
      constexpr bool kBCopiesAll = !C::kAllWavesDq;
      auto copy_tile = [&](int o, int lane_op, bool qtile) __attribute__((always_inline)) {
        if (o < kPW) {
          const int blk = pr + 4 * o;
          if (o + 1 < kPW || blk < kQNI) {
            constexpr int SPR = TileGeom<D>::CPR + 1;
            const int slot = blk * 64 + lane_op;
            const int r = slot / SPR;
            int c = slot - r * SPR;
            c = c < TileGeom<D>::CPR ? c : 0;
            int row = q0_n + r;
            row = row < nb_n - 1 ? row : nb_n - 1;
            dma16((qtile ? p.q : p.dO) + bh_n * N * D, static_cast<unsigned>(row * (2 * D) + 16 * c),
                  smem + (qtile ? C::OFF_Q : C::OFF_DO) + (buf ^ 1) * C::QT + blk * 1024);
          }
        } else if (pr == 0) {
          dma4((qtile ? p.nlse2 : p.neg_delta) + bh_n * p.row_stride + q0_n, row_lane,
               smem + (qtile ? C::OFF_NL : C::OFF_DL) + (buf ^ 1) * 256);
        }
      };
      auto copy_op = [&](int o, int lane_op) __attribute__((always_inline)) { copy_tile(o, lane_op, roleA); };
      Pending pd_n;
      int sem_now = 0;
      if constexpr (roleA) {
        // ---- S = Q K^T (both 32-row blocks), operands kR - 1 slots ahead.
        floatx16 S0, S1;
        // Causal diagonal: S = -inf (P = 0) where the key comes after the query. Row of
        // element r = 4 t + e of block qb: pi(m) = 32 qb + 16 (t / 2) + 2 (t % 2) + 4 e + hi.
        const bool diag = p.causal && j == kv_tile;
        const int mask_thr = kvcol - q0 - hi;
        auto mask_block = [&](int qb, floatx16& S) __attribute__((always_inline)) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int t = r >> 2, e = r & 3;
            if (32 * qb + 16 * (t >> 1) + 2 * (t & 1) + 4 * e < mask_thr) S[r] = -__builtin_inff();
          }
        };
        // P = exp2(s log2(e) S - LSE log2(e)) of elements r, r + 1 of block qb, as a bf16 pair.
        u32x4 P[2][2];
        floatx4 nl[2][4];
        auto softmax2 = [&](int qb, int r, const floatx16& S) __attribute__((always_inline)) {
          const floatx4& n4 = nl[qb][r >> 2];
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r], p.scale_log2, n4[r & 3]));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S[r + 1], p.scale_log2, n4[(r & 3) + 1]));
          P[qb][r >> 3][(r & 7) >> 1] = pack_bf16(p0, p1);
        };
        auto load_nl = [&](int qb) __attribute__((always_inline)) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
            nl[qb][t] = *reinterpret_cast<const LDS_AS floatx4*>(sNL + (qb * 32 + 8 * t + 4 * hi) * 4);
        };
        // S of block 0 with the next step's Q-tile copies between its MFMAs (issued as early
        // as possible: a copy that misses the L2 then still lands before the step ends), S
        // of block 1 with block 0's softmax between its MFMAs (two elements per slot), then
        // block 1's softmax. (Copies placed after block 0 split the loop at a branch, and
        // the compiler then sank block 0's softmax below block 1's MFMAs.)
        int lane_op = 0;
        bf16x8 aq[kR];
#pragma unroll
        for (int i = 0; i < kR - 1; ++i) aq[i] = lds_ld16(sQ, sdp_off(i / DK, i % DK));
        SLOT();
#pragma unroll
        for (int i = 0; i < 2 * DK; ++i) {
          if (i + kR - 1 < 2 * DK) aq[(i + kR - 1) % kR] = lds_ld16(sQ, sdp_off((i + kR - 1) / DK, (i + kR - 1) % DK));
          if (i == 0) load_nl(0);
          if (i == DK / 2) load_nl(1);
          SLOT();  // the operand reads ahead stay ahead of this slot's MFMA
          floatx16& S = i < DK ? S0 : S1;
          if (i % DK == 0)
            mfma32_vab_zero(S, aq[i % kR], kv[0]);
          else
            mfma32_vab(S, aq[i % kR], kv[i % DK]);
          if (i == DK - 1) {
            mfma_result_wait(S0);
            if (diag) mask_block(0, S0);
          }
          if (i >= DK) {
#pragma unroll
            for (int r = 16 * (i - DK) / DK; r < 16 * (i - DK + 1) / DK; r += 2) softmax2(0, r, S0);
          } else {
            // The running sums loaded at the end of the last step have landed before the
            // first copy is issued (the copies are invisible to the compiler's counters).
            if constexpr (!kBCopiesAll) {
              if (i == 0) {
                asm volatile("" : "+v"(ld));
                lane_op = opaque_lane();
              }
#pragma unroll
              for (int o = i * kCopyOps / DK; o < (i + 1) * kCopyOps / DK; ++o) copy_op(o, lane_op);
            }
          }
          SLOT();
        }
        PROF_MARK(kProfSd0);
        // P to the pair's exchange area: block 0 now, block 1 after its softmax.
#pragma unroll
        for (int h = 0; h < 2; ++h) *reinterpret_cast<LDS_AS u32x4*>(sPX + 1024 * h) = P[0][h];
        mfma_result_wait(S1);
        if (diag) mask_block(1, S1);
#pragma unroll
        for (int r = 0; r < 16; r += 2) softmax2(1, r, S1);
#pragma unroll
        for (int h = 0; h < 2; ++h) *reinterpret_cast<LDS_AS u32x4*>(sPX + 1024 * (2 + h)) = P[1][h];
        PROF_MARK(kProfMid0);
        // This pair's P is in LDS: the flag tells the pair's B wave (the LDS writes have
        // completed before the flag is written).
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0) *sFlag = gstep;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        PROF_MARK(kProfBarrierX);
        // ---- dV += P^T dO, with the previous step's dQ block in the first half.
        if (have_prev && !loaded) {
          reduce_wait(pd);
          reduce_load(pd, ld);
          PROF_COUNT(kProfLate);
        }
        PROF_MARK(kProfWait);
#ifdef DASH_REPLAY
        run = ld;
#endif
        pd_n = reduce_prepare(rec_cur);
        sem_now = reduce_poll(pd_n);
        PROF_MARK(kProfDq);
        // The dQ MFMAs run in the first half, so that their stores are acknowledged
        // under the second half's dV MFMAs.
        // QPI dQ MFMAs per dV MFMA over the first NQI dV MFMAs (d = 128: one each over
        // the first half; d = 64: two each over the first half), operands one
        // iteration ahead.
        constexpr int QPI = 2 * KK > 2 * NIT ? 2 : 1;
        constexpr int NQI = KK / QPI;
        bf16x8 bo[kR], aqd[2][QPI];
#pragma unroll
        for (int i = 0; i < kR - 1; ++i) bo[i] = bt_load(sdO, i);
#pragma unroll
        for (int u = 0; u < QPI; ++u)
          if (HAS_DQ) aqd[0][u] = dq_opnd(sdSprev, u);
        SLOT();
#pragma unroll
        for (int jj = 0; jj < 2 * NIT; ++jj) {
          if (jj + kR - 1 < 2 * NIT) bo[(jj + kR - 1) % kR] = bt_load(sdO, jj + kR - 1);
          if (HAS_DQ && jj + 1 < NQI) {
#pragma unroll
            for (int u = 0; u < QPI; ++u) aqd[(jj + 1) & 1][u] = dq_opnd(sdSprev, QPI * (jj + 1) + u);
          }
          SLOT();
          const int qb = jj / NIT, itr = jj % NIT;
          mfma32_acc(acc[itr % DB], as_bf16x8(P[qb][itr / DB]), bo[jj % kR]);
          if (HAS_DQ && jj < NQI) {
#pragma unroll
            for (int u = 0; u < QPI; ++u) dq_mma(ld, QPI * jj + u, aqd[jj & 1][u], kT[QPI * jj + u]);
          }
          if (jj == NQI) {
            mfma_result_wait(ld);
            reduce_store(pd, ld);
          }
          SLOT();
        }
        PROF_MARK(kProfDv0);
        PROF_MARK(kProfLoads);
        if (DET) {
          // Stores (and this step's copies) acknowledged: the previous step's turn is
          // passed on.
          wait_mem_done();
          if (have_prev) reduce_signal(pd);
        } else {
          // The copies have landed before the step-end barrier; the 16 float atomics
          // issued after them stay in flight.
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          __builtin_amdgcn_s_waitcnt(wait_vmcnt(16));
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
        }
        PROF_MARK(kProfReduce);
        const int sem_seen = __builtin_amdgcn_readfirstlane(sem_now);
        loaded = !reduce_needs_turn(pd_n) || sem_seen == pd_n.rank;
        if (loaded) reduce_load(pd_n, ld);
        PROF_MARK(kProfBody);
      } else {
        // ---- The next step's dO-tile copies; dP - D = dO V^T - D (the accumulation
        // starts from -D); the previous step's dQ block in the second half; its stores.
        if (have_prev && !loaded) {
          reduce_wait(pd);
          reduce_load(pd, ld);
          PROF_COUNT(kProfLate);
        }
        PROF_MARK(kProfWait);
        // The running sums have landed before the first copy is issued.
        asm volatile("" : "+v"(ld));
        PROF_MARK(kProfLoads);
#ifdef DASH_REPLAY
        run = ld;
#endif
        const int lane_op = opaque_lane();
        floatx16 dP0, dP1;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          floatx16& x = qb ? dP1 : dP0;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const floatx4 d4 = *reinterpret_cast<const LDS_AS floatx4*>(sDL + (qb * 32 + 8 * t + 4 * hi) * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * t + e] = d4[e];
          }
        }
        bf16x8 ad[kR], aqd[kR];
#pragma unroll
        for (int i = 0; i < kR - 1; ++i) ad[i] = lds_ld16(sdO, sdp_off(i / DK, i % DK));
        SLOT();
#pragma unroll
        for (int i = 0; i < 2 * DK; ++i) {
          if (i + kR - 1 < 2 * DK) ad[(i + kR - 1) % kR] = lds_ld16(sdO, sdp_off((i + kR - 1) / DK, (i + kR - 1) % DK));
          const int kk = i - (2 * DK - KK);
          if (HAS_DQ && kk + kR - 1 >= 0 && kk + kR - 1 < KK)
            aqd[(kk + kR - 1) % kR] = dq_opnd(sdSprev, kk + kR - 1);
          SLOT();
          mfma32_vab(i < DK ? dP0 : dP1, ad[i % kR], kv[i % DK]);
          if (HAS_DQ && kk >= 0) dq_mma(ld, kk, aqd[kk % kR], kT[kk]);
          if (i < DK) {
#pragma unroll
            for (int o = i * kCopyOps / DK; o < (i + 1) * kCopyOps / DK; ++o) copy_op(o, lane_op);
          } else if (kBCopiesAll) {
#pragma unroll
            for (int o = (i - DK) * kCopyOps / DK; o < (i - DK + 1) * kCopyOps / DK; ++o) copy_tile(o, lane_op, true);
          }
          SLOT();
        }
        PROF_MARK(kProfSd0);
        mfma_result_wait(dP0, dP1);
        mfma_result_wait(ld);
        reduce_store(pd, ld);
        PROF_MARK(kProfMid0);
        // Wait for this pair's P (bounded, like the turn waits).
        {
          const long long t0 = wall_clock64();
          int spins = 0;
          while (__builtin_amdgcn_readfirstlane(*sFlag) != gstep) {
            __builtin_amdgcn_s_sleep(1);
            if ((++spins & 63) == 0 && wall_clock64() - t0 > p.timeout_ticks) {
              if (lane == 0) raise_error(p.err, kErrTimeout);
              failed = true;
              break;
            }
          }
        }
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        PROF_MARK(kProfBarrierX);
        // ---- dS = P (dP - D): bf16 pairs in registers, dS^T to LDS; dK += dS^T Q.
        pd_n = reduce_prepare(rec_cur);
        sem_now = reduce_poll(pd_n);
        u32x4 Pw[2][2], dS[2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int h = 0; h < 2; ++h) Pw[qb][h] = *reinterpret_cast<const LDS_AS u32x4*>(sPX + 1024 * (2 * qb + h));
        // dS of elements r, r + 1 of block qb; after the last pair of a row group t, the
        // group's dS^T goes to LDS.
        auto ds2 = [&](int qb, int r) __attribute__((always_inline)) {
          const floatx16& dPx = qb ? dP1 : dP0;
          const unsigned u = Pw[qb][r >> 3][(r & 7) >> 1];
          const float p0 = __builtin_bit_cast(float, u << 16);
          const float p1 = __builtin_bit_cast(float, u & 0xffff0000u);
          dS[qb][r >> 3][(r & 7) >> 1] = pack_bf16(p0 * dPx[r], p1 * dPx[r + 1]);
          if ((r & 3) == 2) {
            const int t = r >> 2;
            u32x2 v2;
            v2[0] = dS[qb][t >> 1][2 * (t & 1)];
            v2[1] = dS[qb][t >> 1][2 * (t & 1) + 1];
            *reinterpret_cast<LDS_AS u32x2*>(sdS + ds_wr_lane + 64 * qb + 16 * t) = v2;
          }
        };
#pragma unroll
        for (int r = 0; r < 16; r += 2) ds2(0, r);
        PROF_MARK(kProfSd1);
        // dK of block 0 with block 1's dS between its MFMAs (two elements per slot), then
        // dK of block 1.
        bf16x8 bq[kR];
#pragma unroll
        for (int i = 0; i < kR - 1; ++i) bq[i] = bt_load(sQ, i);
        SLOT();
#pragma unroll
        for (int jj = 0; jj < 2 * NIT; ++jj) {
          if (jj + kR - 1 < 2 * NIT) bq[(jj + kR - 1) % kR] = bt_load(sQ, jj + kR - 1);
          SLOT();
          const int qb = jj / NIT, itr = jj % NIT;
          mfma32_acc(acc[itr % DB], as_bf16x8(dS[qb][itr / DB]), bq[jj % kR]);
          if (jj < NIT) {
#pragma unroll
            for (int r = 16 * jj / NIT; r < 16 * (jj + 1) / NIT; r += 2) ds2(1, r);
          }
          if (jj == NIT) {
            PROF_MARK(kProfDv0);
            // Stores and copies acknowledged: the previous step's turn is passed on. (The
            // atomic variant waits for the copies only; its atomics stay in flight.)
            if (DET) {
              wait_mem_done();
            } else {
              __atomic_signal_fence(__ATOMIC_SEQ_CST);
              __builtin_amdgcn_s_waitcnt(wait_vmcnt(HAS_DQ ? 16 : 0));
              __atomic_signal_fence(__ATOMIC_SEQ_CST);
            }
            if (have_prev) reduce_signal(pd);
            PROF_MARK(kProfReduce);
          }
          if (jj == NIT + NIT / 2) {
            const int sem_seen = __builtin_amdgcn_readfirstlane(sem_now);
            loaded = !reduce_needs_turn(pd_n) || sem_seen == pd_n.rank;
            if (loaded) reduce_load(pd_n, ld);
          }
          SLOT();
        }
      }
#undef SLOT
      pd = pd_n;
      if constexpr (!roleA) PROF_MARK(kProfBody);
      // Y: dS^T of every pair is visible, the copies have landed, P has been read.
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      PROF_MARK(kProfBarrier);
      rec_cur = rec_nxt;
      rec_nxt = rec_nn;
      mfma_settle(acc);
    }
    // The item's last step: its dQ block and reduction.
    if constexpr (HAS_DQ) {
      if (!loaded) {
        reduce_wait(pd);
        reduce_load(pd, ld);
      }
#ifdef DASH_REPLAY
      run = ld;
#endif
      const LDS_AS char* sdSl = smem + C::OFF_DS + ((par0 + n_steps - 1) & 1) * C::DST;
      bf16x8 a[2];
      a[0] = dq_opnd(sdSl, 0);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) a[(kk + 1) & 1] = dq_opnd(sdSl, kk + 1);
        dq_mma(ld, kk, a[kk & 1], kT[kk]);
        __builtin_amdgcn_sched_barrier(0);
      }
      mfma_result_wait(ld);
      reduce_store(pd, ld);
      wait_mem_done();
      reduce_signal(pd);
      PROF_MARK(kProfFlush);
    }
    par0 = (par0 + n_steps) & 1;
    if (has_next && !roleA) issue_kv(it + 1, par0);

    // Epilogue: dV (A) or dK = s dK (B), bf16, through LDS so that every lane stores
    // 16-byte row chunks. A stages in its 32 rows of the dS^T buffer that the next item's
    // step 0 writes; B in its pair's P exchange area (32 rows x 128 bytes). Both are
    // free from the last step's barrier to the next item's prologue barrier.
    LDS_AS char* stage = roleA ? smem + C::OFF_DS + par0 * C::DST + 32 * pr * kDsStride
                               : smem + C::OFF_PX + pr * C::PXW;
    const int sst = roleA ? kDsStride : 128;
    bf16* g = (roleA ? p.dv : p.dk) + bg * N * D;
    const float mul = roleA ? 1.f : p.scale;
#pragma unroll
    for (int half = 0; half < DB / 2; ++half) {
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 8 * (r >> 2) + 4 * hi + (r & 3);
          *reinterpret_cast<LDS_AS bf16*>(stage + row * sst + 2 * (32 * e2 + l32)) =
              static_cast<bf16>(acc[2 * half + e2][r] * mul);
        }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int chunk = lane + 64 * k, row = chunk >> 3, c16 = chunk & 7;
        const u32x4 v = *reinterpret_cast<const LDS_AS u32x4*>(stage + row * sst + 16 * c16);
        const int kvr = kv0 + 32 * pr + row;
        if (kvr < nb) *reinterpret_cast<u32x4*>(g + static_cast<int64_t>(kvr) * D + 64 * half + 8 * c16) = v;
      }
    }
    PROF_MARK(kProfEpi);
  }
  PROF_STORE(p, w, 8);
}

// DET: ordered reduction inside one XCD's L2 (every dQ tile's contributors share an
// XCD), or float atomics; PART (with DET): every contribution to its own slot of the
// per-tile partials buffer, no turns (a separate kernel adds them); FUSED (with DET, not
// PART): the last contributor of every dQ block writes bf16 dQ (p.dq) instead of its
// final fp32 sum. One kernel each, so that no instance carries another's code.
template <int D, bool DET, bool PART, bool FUSED>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
bwd_pair_kernel(BwdParams p) {
  using C = PairCfg<D>;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  LDS_AS int* sMisc = reinterpret_cast<LDS_AS int*>(smem + C::OFF_MISC);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  if (tid < 4) sMisc[4 + tid] = 0;  // P-ready flags of the pairs (no step yet)
  __syncthreads();
  const int worker = sMisc[0];
  if (worker < 0) return;
  if (w < 4)
    pair_body<D, DET, true, PART, FUSED>(p, smem, worker, w);
  else
    pair_body<D, DET, false, PART, FUSED>(p, smem, worker, w);
}

template <int D>
static hipError_t launch_pair_t(const BwdParams& prm, int grid, hipStream_t stream) {
  using C = PairCfg<D>;
  const int shmem = C::BYTES;
  auto fn = prm.deterministic == 3 ? bwd_pair_kernel<D, true, true, false>
            : prm.deterministic && prm.dq ? bwd_pair_kernel<D, true, false, true>
            : prm.deterministic   ? bwd_pair_kernel<D, true, false, false>
                                  : bwd_pair_kernel<D, false, false, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, shmem);
  if (e != hipSuccess) return e;
  BwdParams local = prm;
  void* args[] = {&local};
  return launch_resident(reinterpret_cast<const void*>(fn), grid, C::NT, shmem, args, stream);
}

hipError_t launch_pair_d128(const BwdParams& prm, int grid, hipStream_t stream) {
  return launch_pair_t<128>(prm, grid, stream);
}

hipError_t launch_pair_d64(const BwdParams& prm, int grid, hipStream_t stream) {
  return launch_pair_t<64>(prm, grid, stream);
}

}  // namespace dash
