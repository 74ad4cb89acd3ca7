// Internal interface between the host API and the HIP kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>

namespace dash {

// Device error word values (match dash_status in include/dash.h).
constexpr int kErrTimeout = -6;
constexpr int kErrPlacement = -7;

struct PreParams {
  const __bf16* o;
  const __bf16* dO;
  const float* lse;    // [rows] natural-log LSE of the scaled scores
  float* neg_delta;    // [B*H][row_stride] -D = -rowsum(dO * O); 0 past N
  float* nlse2;        // [B*H][row_stride] -LSE * log2(e); -inf past N
  int64_t rows;        // B * H * N
  int N;
  int row_stride;      // N rounded up to the tile
  int* sem;            // ordering semaphores to clear
  int64_t sem_count;
  int* ctr;            // XCD slot counters to clear
  int64_t ctr_count;
  int* err;            // the call's device error word, cleared here
  float* dqacc_zero;   // non-null: clear this fp32 buffer (atomic variant)
  int64_t zero_count;  // elements, multiple of 4
  const int* seqlens;  // non-null: rows of batch b at or past seqlens[b] are padding
  int H;               // query heads (batch of a row = row / N / H)
};

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dO;
  const float* nlse2;  // [B*H][row_stride] -LSE * log2(e); -inf past N
  const float* neg_delta;  // [B*H][row_stride] -D = -rowsum(dO * O); 0 past N
  __bf16* dk;
  __bf16* dv;
  float* dqacc;        // fp32 dQ accumulator (layouts described at kDqBlock)
  int* sem;
  int* ctr;
  int* err;            // the call's device error word (in the workspace; 0 = no error)
  const int* worker_begin;
  const int4* items;
  const int4* tasks;
  const int4* steps;   // per 64-row step in task order: {b * H + h, first Q row, rank, last}; 2 zero records follow
  int B, H, Hkv, N;
  int sem_stride;      // semaphores per (b, h): kSemPerStep per 64-row Q step, padded
  int row_stride;      // rows per (b, h) of nlse2, neg_delta and dqacc: N rounded up to the tile
  float scale;         // softmax scale s
  float scale_log2;    // s * log2(e)
  int causal;
  int deterministic;
  int xcd_local;       // 1: every dQ tile's contributors share one XCD (L2)
  int num_xcd;
  int cus_per_xcd;
  long long timeout_ticks;  // wall-clock ticks before a wait gives up
  unsigned long long* prof; // profiling builds (DASH_PROFILE): per-wave phase cycle counters, or null
  float* replay;            // replay builds (DASH_REPLAY): dump of every ordered dQ partial, or null
  int replay_ranks;         // replay builds: rank slots per dQ block in the dump (KV tiles per head)
  const int* seqlens;       // non-null: batch b has seqlens[b] rows (<= N, the row stride of q, k, ...)
  // Ordered reduction in the two-waves kernel: non-null = the last contributor of every
  // dQ block writes bf16(scale * final sum) straight into dq [B*H][N][d] (rows past a
  // batch's length untouched) instead of storing the final fp32 sum, so no cast kernel
  // follows. Null: every sum goes to dqacc, and dq_cast_blocks_kernel writes dq.
  __bf16* dq;
};

// Forward kernel (O and the natural-log LSE from Q, K, V).
struct FwdParams {
  const __bf16* q;   // [B, H, N, d]
  const __bf16* k;   // [B, Hkv, N, d]
  const __bf16* v;   // [B, Hkv, N, d]
  __bf16* o;         // [B, H, N, d]
  float* lse;        // [B, H, N]
  int B, H, Hkv, N;
  int n_qt;          // 128-row Q tiles per head
  int causal;
  float scale_log2;  // softmax scale * log2(e)
};

// dQ pass of the two-pass variant.
struct DqParams {
  const __bf16* q;          // [B, H, N, d]
  const __bf16* k;          // [B, Hkv, N, d]
  const __bf16* v;          // [B, Hkv, N, d]
  const __bf16* dO;         // [B, H, N, d]
  const float* nlse2;       // [B*H][row_stride] -LSE * log2(e)
  const float* neg_delta;   // [B*H][row_stride] -D
  __bf16* dq;               // [B, H, N, d]
  const int* seqlens;       // rows of each batch (variable-length batches), or null: N
  int B, H, Hkv, N;
  int row_stride;
  int n_qt;                 // 128-row Q tiles per head
  int causal;
  float scale;              // softmax scale s
  float scale_log2;         // s * log2(e)
  const int* err_in;        // the call's error word, final once the main kernel is done
  int* status_out;          // the stream's status slot: receives *err_in (block 0)
};

// fp32 dQ accumulator layouts (rows per (b, h) padded to row_stride).
// - Ordered variant, block layout: the rows are cut into 32-row blocks and the d
//   columns into 32-column blocks; block (qblk, db) is kDqBlock floats at
//   ((bh * row_stride / 32 + qblk) * d / 32 + db) * kDqBlock, in the order of a 32x32
//   MFMA accumulator: element r = 4 i + e (i, e in 0..3) of lane l (0..63) is float
//   256 i + 4 l + e, and it belongs to row 16 (i / 2) + 2 (i % 2) + l / 32 + 4 e, column
//   l % 32 of the block. (Rows are in the permuted order in which the kernel's dS
//   operand visits them.) A wave then moves one block with four 1 KiB accesses.
// - Atomic variant: row-major [bh][row_stride][d], so that the per-element float atomics
//   of a wave hit whole cache lines.
// - Per-tile partials (deterministic = 3): no accumulator; every contribution has its own
//   slot of 2 (64 / 32) x (d / 32) blocks (one 64-row step of one Q tile from one KV tile),
//   in the same block order. Slots of a (b, h) are ordered by Q tile j, then the step's
//   place in the tile, then the contribution's rank; Q tile j has n contributions (full
//   mask) or j + 1 (causal), so a head has steps_per_tile x n^2 or steps_per_tile x
//   n (n + 1) / 2 slots (partial_slot below).
constexpr int kDqBlock = 32 * 32;

// Slot of the per-tile partial of head bh (= b * H + h), 64-row step starting at Q row
// q0, contribution `rank`, for n tiles of `tile` rows per head.
__host__ __device__ inline int64_t partial_slot(int64_t bh, int q0, int rank, int n, int tile, int causal) {
  const int subs = tile / 64;
  const int j = q0 / tile;
  const int sub = (q0 % tile) / 64;
  const int64_t per_head = (causal ? int64_t(n) * (n + 1) / 2 : int64_t(n) * n) * subs;
  const int64_t before = causal ? int64_t(j) * (j + 1) / 2 : int64_t(j) * n;  // slots of earlier Q tiles / subs
  const int cnt = causal ? j + 1 : n;
  return bh * per_head + before * subs + int64_t(sub) * cnt + rank;
}

// Ordering semaphores per 64-row Q step of a (b, h): one per wave of the largest
// workgroup (each wave reduces its own dQ blocks and passes its own turn).
constexpr int kSemPerStep = 8;

// Phase counters of a profiling build, per wave: [grid][NW][kProfSlots] of 64-bit cycles
// (s_memtime) or counts.
constexpr int kProfSlots = 20;
enum ProfSlot {
  kProfBody = 0,     // dV/dK of the second block (the step's last MFMA phase)
  kProfBarrier = 1,  // the step barrier
  kProfDq = 2,       // dQ turn bookkeeping: task record and accumulator addresses
  kProfWait = 3,     // waiting for the dQ turn (semaphore)
  kProfReduce = 4,   // waiting for this wave's copies at the step's end
  kProfItem = 5,     // the step's first LDS reads issued and its running sums landed
  kProfBarrierX = 5, // (two-waves kernel) the mid-step barrier
  kProfSteps = 6,    // number of steps
  kProfTotal = 7,    // whole kernel
  kProfSd0 = 8,      // S/dP of the first block (with dQ MFMAs), from the accumulator loads on
  kProfMid0 = 9,     // stores of the first dQ blocks, mask
  kProfSd1 = 10,     // S/dP of the second block with the first block's softmax
  kProfMid1 = 11,    // stores of the other dQ blocks, their acknowledgement, turn passed on,
                     // next step's copies issued
  kProfDv0 = 12,     // dV/dK of the first block with the second block's softmax
  kProfLoads = 13,   // accumulator loads issued at the step's start (after a late turn)
  kProfLate = 14,    // number of steps whose turn had not come at the poll
  kProfPoll = 15,    // reading the polled turn word
  kProfPro = 16,     // item prologue (K, V, first tiles, K^T operands)
  kProfFlush = 17,   // the item's last reduction
  kProfEpi = 18,     // item epilogue (dK, dV stores)
};

// Launches a persistent grid whose workgroups wait for each other (the ordered dQ
// reduction), so all `grid` workgroups must be resident at once. The device must hold
// that many workgroups of `fn` at a time (occupancy per CU times CUs, cached per kernel
// and device), else hipErrorCooperativeLaunchTooLarge is returned and nothing is
// launched. The launch itself is an ordinary one: on an otherwise idle device every
// workgroup is placed at once; a kernel of another stream that holds CUs only delays
// the start of some workgroups, which the kernels' bounded waits tolerate up to their
// timeout. (A cooperative launch would add nothing the kernels use: they never
// synchronise the whole grid.)
inline hipError_t launch_resident(const void* fn, int grid, int threads, int shmem, void** args,
                                  hipStream_t stream) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> capacity;  // (kernel, device) -> workgroups
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int cap = 0;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = capacity.find({fn, dev});
    if (it != capacity.end()) {
      cap = it->second;
    } else {
      int per_cu = 0, cus = 0;
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, threads, shmem);
      if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
      cap = per_cu * cus;
      capacity.emplace(std::make_pair(fn, dev), cap);
    }
  }
  if (grid > cap) return hipErrorCooperativeLaunchTooLarge;
  return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, shmem, stream);
}

// Main kernel for head dimension d and a workgroup of nw waves (one translation unit each).
hipError_t launch_main_d64_nw2(const BwdParams& prm, int grid, hipStream_t stream);
hipError_t launch_main_d64_nw4(const BwdParams& prm, int grid, hipStream_t stream);
hipError_t launch_main_d128_nw2(const BwdParams& prm, int grid, hipStream_t stream);
hipError_t launch_main_d128_nw4(const BwdParams& prm, int grid, hipStream_t stream);
// Two-waves-per-SIMD main kernel (d = 128, 128-row tiles, ordered XCD-local or atomic
// reduction; 8 waves per workgroup).
hipError_t launch_pair_d128(const BwdParams& prm, int grid, hipStream_t stream);
hipError_t launch_pair_d64(const BwdParams& prm, int grid, hipStream_t stream);
inline hipError_t launch_main(const BwdParams& prm, int d, int nw, int grid, hipStream_t stream) {
  if (d == 64 && nw == 2) return launch_main_d64_nw2(prm, grid, stream);
  if (d == 64 && nw == 4) return launch_main_d64_nw4(prm, grid, stream);
  if (d == 128 && nw == 2) return launch_main_d128_nw2(prm, grid, stream);
  if (d == 128 && nw == 4) return launch_main_d128_nw4(prm, grid, stream);
  return hipErrorInvalidValue;
}
hipError_t launch_preprocess(const PreParams& prm, int d, int grid, hipStream_t stream);
// The last kernel of a backward call copies the call's error word (final by then: the
// main kernel precedes it on the stream) into the stream's status slot, which
// dash_last_kernel_error reads.
struct StatusCopy {
  const int* err_in;
  int* status_out;
};
// Copies the call's error word into the stream's status slot (one thread), for calls
// whose main kernel wrote dQ itself.
hipError_t launch_status_copy(StatusCopy sc, hipStream_t stream);
// dQ = bf16(scale * dqacc) for rows < N, from the ordered variant's block layout.
hipError_t launch_dq_cast_blocks(const float* acc, void* dq, int64_t heads, int N, int row_stride, int d, float scale,
                                 StatusCopy sc, hipStream_t stream, const int* seqlens = nullptr, int H = 1);
// dQ = bf16(scale * dqacc) for rows < N, from the atomic variant's row-major layout.
hipError_t launch_dq_cast(const float* acc, void* dq, int64_t heads, int N, int row_stride, int d, float scale,
                          StatusCopy sc, hipStream_t stream, const int* seqlens = nullptr, int H = 1);
// dQ = bf16(scale * sum of the per-tile partials), rank order, rows < N (deterministic = 3).
hipError_t launch_dq_consolidate(const float* parts, void* dq, int64_t heads, int N, int row_stride, int tile, int d,
                                 int causal, float scale, StatusCopy sc, hipStream_t stream);
hipError_t launch_topology_probe(int* out, int grid, hipStream_t stream);
hipError_t launch_fwd(const FwdParams& prm, int d, hipStream_t stream);
hipError_t launch_dq_pass(const DqParams& prm, int d, hipStream_t stream);

}  // namespace dash
