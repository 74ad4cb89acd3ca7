/*
 * dash.h -- C ABI of the deterministic attention backward for AMD Instinct MI355X (gfx950).
 *
 * The operation (DASH paper, arXiv 2601.21824, section 2.1; "Writing an Attention
 * Kernel", section "In the real world"): given the forward inputs Q, K, V, the
 * forward output O, the upstream gradient dO and the forward's per-row
 * log-sum-exp, compute dQ, dK, dV of softmax attention by recomputing the
 * probabilities tile by tile. KV tiles are spread over compute units; each CU keeps
 * its KV tile's dK/dV in registers (reduction over the query axis, local), while
 * the dQ partial sums of one query tile arrive from many CUs and are added in a
 * fixed order (reduction over the key axis, global). The order is the one the
 * selected schedule defines (section 3): naive (ascending KV index, the
 * FlashAttention-3 deterministic baseline), descending Q-tile iteration (3.3),
 * shift scheduling (3.4, full mask) or symmetric shift (3.4, causal mask).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are dense, row-major, bf16 unless stated:
 *     q, o, dO, dq : [B, H,   N, d]
 *     k, v, dk, dv : [B, Hkv, N, d]
 *     lse          : [B, H, N] float32, natural-log log-sum-exp of the *scaled*
 *                    scores softmax_scale * q.k of each query row.
 *   Query head h reads key/value head h / (H / Hkv) (grouped-query attention).
 *   dk and dv of a key/value head sum the contributions of all its query heads.
 * - The causal mask is top-left aligned: key k is visible to query q iff k <= q.
 * - d must be 64 or 128. Any N >= 1 is accepted (the last tile is partial).
 * - Every pointer of dash_attn_bwd is a device pointer owned by the caller; the
 *   library never frees or retains it. Outputs are overwritten, not accumulated.
 * - `stream` is a hipStream_t (0 = the null stream). Calls return after enqueueing.
 * - All argument checks run before anything is enqueued: on an error return no
 *   kernel is launched and the outputs are untouched.
 * - The library owns, per device: a schedule-table cache for dash_attn_bwd (built on
 *   the first call for a given shape, mask, schedule and placement; that first call
 *   allocates the table and copies it to the device synchronously, later calls with the
 *   same key neither allocate nor synchronise); a pinned host staging ring (64 MiB,
 *   allocated on the first call on the device) from which dash_attn_bwd_varlen copies
 *   its per-call table into the caller's workspace in stream order; and a pinned host
 *   word for dash_last_kernel_error. All live until the process ends. Host state is
 *   guarded by a mutex; calls from several host threads are safe, but two calls that
 *   share a workspace must not overlap.
 * - Kernel-side errors (a bounded wait that timed out, a workgroup on an unexpected
 *   XCD slot) are written to an error word inside the call's workspace, which the call
 *   itself clears in stream order before its kernels run: an error never leaks into a
 *   later call. The call's last kernel copies the word into a status slot of the
 *   stream, which dash_last_kernel_error(stream) reads.
 */
#ifndef DASH_H
#define DASH_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (negative = error). */
typedef enum {
  DASH_OK = 0,
  DASH_ERR_INVALID_ARG = -1,   /* null pointer, bad size, H % Hkv != 0, ...          */
  DASH_ERR_UNSUPPORTED = -2,   /* d not in {64,128}; schedule not defined for mask   */
  DASH_ERR_WORKSPACE = -3,     /* workspace smaller than dash_attn_bwd_workspace_size */
  DASH_ERR_NOT_CORESIDENT = -4,/* the persistent grid cannot be resident at once     */
  DASH_ERR_HIP = -5,           /* a HIP runtime call failed                           */
  DASH_ERR_TIMEOUT = -6,       /* a kernel's ordered-reduction wait timed out         */
  DASH_ERR_PLACEMENT = -7      /* the workgroups did not land on the CUs the table expects */
} dash_status;

typedef enum { DASH_MASK_FULL = 0, DASH_MASK_CAUSAL = 1 } dash_mask;

/* Tile-to-CU schedules (DASH, section 3). shift is defined for the full mask only,
 * sym_shift for the causal mask only (with an even number of KV tiles per head).
 * DASH_SCHED_AUTO runs the valid schedule (naive, descending, and shift for the full
 * mask or sym_shift for the causal mask) with the smallest makespan under a DAG cost
 * model of the tables for the device's topology (section 3.1 graph, per-task costs
 * measured on MI355X, cross-XCD reductions priced apart); dash_schedule_resolve names
 * it. On the paper's benchmark grid that is shift (full) and sym_shift (causal). */
typedef enum {
  DASH_SCHED_NAIVE = 0,
  DASH_SCHED_DESCENDING = 1,
  DASH_SCHED_SHIFT = 2,
  DASH_SCHED_SYM_SHIFT = 3,
  DASH_SCHED_AUTO = 4
} dash_schedule;

/* CU-group placement (DASH paper, section 3: "n KV tiles = n SMs; otherwise refine or
 * aggregate heads"). A KV head's group has one lane per KV tile (one per tile pair for
 * the symmetric shift); when it has more lanes than one XCD has CUs:
 *   DASH_PLACEMENT_AGGREGATE (default): the group stays on one XCD and each CU runs
 *     several lanes one after another, so every dQ chain stays in one L2;
 *   DASH_PLACEMENT_SPREAD: the group spans as many XCDs as it needs, one lane per CU
 *     (the paper's n-SM layout); dQ chains then cross XCDs and use device-scope
 *     ordering. Smaller groups are placed the same way under both. */
typedef enum { DASH_PLACEMENT_AGGREGATE = 0, DASH_PLACEMENT_SPREAD = 1 } dash_placement;

/* Sets the placement used by later calls (library-wide, thread-safe; tables are cached
 * per placement). Returns DASH_OK, or DASH_ERR_INVALID_ARG for another value. */
int dash_set_placement(int placement);

/* Main backward kernel. The one-wave-per-SIMD kernel gives each of 4 waves per CU 32 KV
 * rows and all five contractions. The two-waves-per-SIMD kernel gives the same 32 rows
 * to a pair of waves that split the contractions by role (S, P, dV and dP, dS, dK; one
 * dQ block each), so that two waves share every SIMD. The latter covers 128-row tiles
 * (N >= 512) with deterministic = 0 or 1 (dQ chains inside one XCD); other calls use the
 * former under every setting. DASH_KERNEL_AUTO picks the one measured faster: the
 * two-waves kernel wherever it applies. Both give results within the same tolerance;
 * their bits differ (dS is formed from the bf16 P in the two-waves kernel), and each is
 * bitwise reproducible on its own. */
typedef enum {
  DASH_KERNEL_AUTO = 0,
  DASH_KERNEL_ONE_WAVE_PER_SIMD = 1,
  DASH_KERNEL_TWO_WAVES_PER_SIMD = 2
} dash_kernel;

/* Sets the main kernel used by later calls (library-wide, thread-safe). Returns DASH_OK,
 * or DASH_ERR_INVALID_ARG for another value. */
int dash_set_kernel(int kernel);

/* Sets the bound of every wait inside the backward kernels of later calls (the ordered
 * reduction's turn waits and the two-waves kernel's in-step handoff), in microseconds,
 * 0 .. 3.6e9 (default 5 000 000 = 5 s; library-wide, thread-safe). A wait that runs past
 * it (checked every few dozen polls, so 0 means "a few dozen polls") records
 * DASH_ERR_TIMEOUT for dash_last_kernel_error and gives up; every other wave then stops
 * waiting too, the kernels drain, and the outputs of that call are undefined. For
 * callers with a watchdog of their own and for tests of the error path. Returns DASH_OK,
 * or DASH_ERR_INVALID_ARG for a value outside the range. */
int dash_set_wait_timeout(long long microseconds);

/* Bytes of caller-provided device workspace dash_attn_bwd needs for this shape:
 * an fp32 dQ accumulator of B*H*R*d floats and two fp32 row-term arrays of B*H*R
 * floats (-D with D = rowsum(dO*O), and -LSE*log2(e)), where R is N rounded up to the
 * tile (dash_tile_size), plus the int32 ordering semaphores, XCD slot counters and the
 * call's error word. The contents are the library's own between calls (the accumulator
 * is kept in the matrix-core accumulator order, not row-major). Returns 0 for invalid
 * sizes. */
size_t dash_attn_bwd_workspace_size(int B, int H, int Hkv, int N, int d);

/* Bytes of workspace dash_attn_bwd needs with deterministic = 3 (per-tile partials) for
 * this shape and mask: in place of the accumulator, one fp32 slot of 64 x d floats per
 * (batch, query head, 64-row query step, contributing KV tile), i.e.
 * B*H*(tile/64)*n^2 slots for the full mask and B*H*(tile/64)*n(n+1)/2 for the causal
 * mask (n = ceil(N / tile)); e.g. 2.1 GB at B=8, H=16, N=2048, d=128, full mask. Returns 0
 * for invalid sizes or mask. */
size_t dash_attn_bwd_partials_workspace_size(int B, int H, int Hkv, int N, int d, int mask);

/* Bytes of workspace dash_attn_bwd_varlen needs for a padded batch of these sizes: the
 * dash_attn_bwd workspace plus a region for the call's schedule table (an upper bound
 * for any batch lengths: B*H*ceil(N/tile)^2 tasks). Returns 0 for invalid sizes. */
size_t dash_attn_bwd_varlen_workspace_size(int B, int H, int Hkv, int N, int d);

/* The backward pass (DASH, section 2.1; the schedules of section 3).
 * deterministic = 1: dQ partial sums are added in the schedule's fixed order; the
 *   result is bitwise identical from run to run.
 * deterministic = 0: dQ partial sums are added with floating-point atomics
 *   (completion order, not reproducible; kept for comparison, section 1). The
 *   schedule still sets the tile order.
 * deterministic = 2: two-pass variant, the alternative the paper contrasts with its
 *   design (section 5): the main kernel computes dK and dV only, and a second kernel
 *   walks all key tiles for each query tile, recomputing S and dP, with dQ kept in
 *   registers (deterministic, no cross-CU reduction). The schedule sets the tile
 *   order of the dK/dV pass.
 * deterministic = 4: the bitwise-reproducible mode measured faster on MI355X for the
 *   shape, 1 or 2 (dash_deterministic_resolve names it): the two-pass variant for
 *   grouped-query attention with 8 or more query heads per KV head, or 4 or more with the
 *   causal mask at d = 128 and N >= 4096 (where the ordered reduction has few lanes and a
 *   large hot set per XCD); the ordered reduction otherwise. The workspace is the same.
 * deterministic = 3: per-tile partials, the other deterministic alternative of section
 *   5 (FlashAttention-2 style): every dQ contribution of every KV tile is written to its
 *   own fp32 slot, with no waits, and a separate kernel adds each query step's slots in
 *   the schedule's rank order (fp32, from +0) and writes bf16 dQ. Bitwise reproducible;
 *   the workspace is dash_attn_bwd_partials_workspace_size (far larger). Not with
 *   dash_attn_bwd_varlen (DASH_ERR_UNSUPPORTED there).
 * softmax_scale must be finite and > 0 (1/sqrt(d) for standard attention).
 * B == 0 or N == 0 is a no-op that returns DASH_OK.
 * Errors: DASH_ERR_INVALID_ARG, _UNSUPPORTED, _WORKSPACE, _NOT_CORESIDENT, _HIP.
 * Kernel-side failures (a timed-out wait) are reported by dash_last_kernel_error(stream). */
int dash_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                  const void* dO, const float* lse,
                  void* dq, void* dk, void* dv,
                  int B, int H, int Hkv, int N, int d, float softmax_scale,
                  int mask, int schedule, int deterministic,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Same as dash_attn_bwd, and additionally records the hipEvent_t main_start before
 * and main_stop after the main backward kernel on `stream` (either may be null),
 * so callers can time that kernel alone. */
int dash_attn_bwd_timed(const void* q, const void* k, const void* v, const void* o,
                        const void* dO, const float* lse,
                        void* dq, void* dk, void* dv,
                        int B, int H, int Hkv, int N, int d, float softmax_scale,
                        int mask, int schedule, int deterministic,
                        void* workspace, size_t workspace_bytes, void* stream,
                        void* main_start, void* main_stop);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): dash_attn_bwd without a workspace
 * argument. Its workspace and its schedule table live in a static device array of the
 * library, 64 MiB per device, held from the loading of the library until the process
 * ends: 8 MiB for schedule tables and 56 MiB of workspace, so the call accepts shapes
 * whose dash_attn_bwd_workspace_size is at most 56 MiB (B*H*ceil(N/tile)*tile*d*4 bytes
 * of accumulator plus small row terms; e.g. B=2, H=16, N=2048, d=128) and returns
 * DASH_ERR_WORKSPACE for larger ones. deterministic = 0, 1 or 2 (3, the per-tile
 * partials, returns DASH_ERR_UNSUPPORTED). The call allocates nothing: no hipMalloc,
 * hipFree or allocating HIP call. The first call for a shape builds its schedule table
 * on the host and copies it into the array on `stream` (later calls with that shape copy
 * nothing; tables of older shapes are dropped when the table part is full). Every call
 * on a device shares that device's array, which keeps the last call's contents: calls
 * that overlap on one device (e.g. on two streams) race and give undefined results;
 * calls ordered on one stream are safe. Results are bitwise those of dash_attn_bwd with
 * the same arguments. dash_last_kernel_error(stream) reports its kernel-side status.
 * Other errors as dash_attn_bwd. */
int dash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                          const void* dO, const float* lse,
                          void* dq, void* dk, void* dv,
                          int B, int H, int Hkv, int N, int d, float softmax_scale,
                          int mask, int schedule, int deterministic, void* stream);

/* The forward pass ("Writing an Attention Kernel", Steps 1 and 2): O = softmax(s Q K^T) V
 * and lse = the natural-log log-sum-exp of each query row's scaled scores s q.k, i.e.
 * the o and lse that dash_attn_bwd takes. Key tiles are visited in ascending order with
 * an online softmax (running maximum and sum per row); the result is deterministic.
 * q: [B, H, N, d], k, v: [B, Hkv, N, d] bf16 (read); o: [B, H, N, d] bf16 and
 * lse: [B, H, N] float32 (written). Device pointers owned by the caller; q, k, v, o
 * 16-byte aligned, lse 4-byte aligned. Same size, mask and scale rules as dash_attn_bwd;
 * no workspace and no schedule. B == 0 or N == 0 is a no-op that returns DASH_OK.
 * Errors (before anything is enqueued): DASH_ERR_INVALID_ARG, _UNSUPPORTED; DASH_ERR_HIP
 * if the launch fails. */
int dash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                  int B, int H, int Hkv, int N, int d, float softmax_scale, int mask, void* stream);
/* Kernel-side status of the last backward call (dash_attn_bwd and its variants) that
 * ran kernels on `stream` (a hipStream_t; 0 = the null stream) on the current device:
 * DASH_OK, DASH_ERR_TIMEOUT or DASH_ERR_PLACEMENT. Synchronizes that stream only. Each
 * call's last kernel copies the call's error word into a library-owned status slot of
 * its stream (4096 slots per device, handed out per stream in order and reused round
 * robin beyond that), so the status survives the call's workspace. DASH_OK when no
 * backward call ran on the stream; DASH_ERR_HIP if the copy or the synchronization
 * fails. Reading does not clear the status (the stream's next call overwrites it). */
int dash_last_kernel_error(void* stream);

/* Human-readable name of a status code (static storage; never null). */
const char* dash_status_string(int status);

/* KV/Q tile edge (rows) the library uses for this sequence length: 64 when N < 512,
 * else 128. The schedules work on a square grid of ceil(N / tile) tiles per head. */
int dash_tile_size(int N);

/* Host-only export of the schedule table, for checking (no GPU work).
 * The table is built for `num_xcd` L2 domains of `cus_per_xcd` compute units each
 * (the GPU library uses the topology it measures on the device).
 * Writes up to `capacity` records of 7 ints into `records`:
 *   (worker, b, h, g, i, j, rank)
 * in worker order and, within a worker, in execution order. worker = xcd *
 * cus_per_xcd + slot; i = KV tile, j = Q tile, rank = position of this task in the
 * reduction order of dQ tile (b, h, j). *count receives the number of records (also
 * when capacity is too small, in which case DASH_ERR_WORKSPACE is returned and
 * nothing is written). *xcd_local (may be null) receives 1 when every dQ tile's
 * contributors sit on one L2 domain. DASH_SCHED_AUTO is resolved as by
 * dash_schedule_resolve with d = 128. Errors: as dash_attn_bwd's argument checks. */
int dash_schedule_table(int B, int H, int Hkv, int N, int mask, int schedule,
                        int num_xcd, int cus_per_xcd,
                        int* records, long long capacity, long long* count, int* xcd_local);

/* Variable-length batches (a training batch often holds sequences of different
 * lengths; the DASH paper's section 4.1 benchmarks one length at a time). Same call as
 * dash_attn_bwd on the padded layout: q, o, dO, dq [B,H,N,d], k, v, dk, dv [B,Hkv,N,d],
 * lse [B,H,N], where batch b holds seqlens[b] rows (a HOST array of B ints, 1 <=
 * seqlens[b] <= N; N is the padded length and the row stride). Batch b's backward is
 * exactly the attention backward of its first seqlens[b] rows (causal: top-left
 * aligned within the batch); rows at or past seqlens[b] of dq, dk and dv are left
 * unchanged, and those rows of the inputs are never read as data. The schedule applies
 * per batch (DASH_SCHED_AUTO: the model's choice at each batch's length).
 * Every deterministic mode, tile size and main kernel is supported. The workspace is
 * dash_attn_bwd_varlen_workspace_size(B, H, Hkv, N, d): the call's table (built on the
 * host, its image cached for the 64 most recent length vectors) is copied into it on
 * `stream` from the library's pinned staging ring, so the call allocates no device
 * memory and does not wait for the device (except when more tables than the ring holds
 * are still queued, or one table is larger than the ring, which then grows).
 * Errors: as dash_attn_bwd, and
 * DASH_ERR_INVALID_ARG for a null seqlens or a length outside [1, N]; symmetric shift
 * needs an even tile count (of the padded length's tile size) in every batch. */
int dash_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dO,
                         const float* lse, void* dq, void* dk, void* dv,
                         int B, int H, int Hkv, int N, int d, const int* seqlens,
                         float softmax_scale, int mask, int schedule, int deterministic,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Host-only export of the table dash_attn_bwd_varlen runs for these batch lengths
 * (seqlens: B host ints in [1, N]), in the records of dash_schedule_table;
 * DASH_SCHED_AUTO resolves per batch as in dash_attn_bwd_varlen with d = 128. */
int dash_schedule_table_varlen(int B, int H, int Hkv, int N, const int* seqlens, int mask, int schedule,
                               int num_xcd, int cus_per_xcd,
                               int* records, long long capacity, long long* count, int* xcd_local);

/* Hardware-aware schedule model (DASH paper, section 3.1 "Graph Construction": every
 * task is a compute edge c then a reduction edge r on its CU, the reductions into one dQ
 * tile follow each other in rank order; section 4.2: synchronising through a remote L2
 * segment costs more than through the local one). Host-only, no GPU work.
 * Builds the table of `schedule` for `num_xcd` L2 domains of `cus_per_xcd` CUs (the
 * current placement) and writes into *makespan the longest path of its DAG when a task
 * costs c, a reduction costs r_remote if the previous reduction into its dQ tile ran on
 * another L2 domain and r_local otherwise (any time unit). DASH_SCHED_AUTO is resolved
 * first as by dash_schedule_resolve with d = 128. Errors: as dash_schedule_table, and
 * DASH_ERR_INVALID_ARG for negative or non-finite costs or a null makespan. */
int dash_schedule_makespan(int B, int H, int Hkv, int N, int mask, int schedule,
                           int num_xcd, int cus_per_xcd,
                           double c, double r_local, double r_remote, double* makespan);

/* The mode dash_attn_bwd runs for `deterministic` (host-only): 0 .. 3 are returned
 * unchanged after the argument checks; 4 becomes 1 or 2 as described at dash_attn_bwd.
 * Returns the mode (>= 0) or a dash_status code (< 0) for invalid arguments. */
int dash_deterministic_resolve(int B, int H, int Hkv, int N, int d, int mask, int deterministic);

/* The schedule dash_attn_bwd runs for `schedule` (host-only): a concrete schedule is
 * returned unchanged after the argument checks; DASH_SCHED_AUTO becomes the valid
 * schedule (naive, descending, and shift for the full mask or symmetric shift for the
 * causal mask) with the smallest dash_schedule_makespan under costs measured on MI355X
 * for head dimension d (task compute, reduction inside one XCD, reduction across XCDs),
 * ties to shift / symmetric shift. Returns the schedule (>= 0) or a dash_status code
 * (< 0) for invalid arguments, as dash_attn_bwd's checks. */
int dash_schedule_resolve(int B, int H, int Hkv, int N, int d, int mask, int schedule,
                          int num_xcd, int cus_per_xcd);

#ifdef __cplusplus
}
#endif

#endif /* DASH_H */
