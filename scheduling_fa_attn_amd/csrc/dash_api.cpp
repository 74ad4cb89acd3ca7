// Host side of the C ABI declared in include/dash.h: argument checks, per-device state
// (measured XCD topology, device error word, schedule-table cache) and kernel launches.
#include "dash.h"
#include "dash_replay.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <deque>
#include <list>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "kernels.h"
#include "schedule.h"

namespace {

using dash::Sched;

constexpr int kCtrInts = 16 * 64;  // one 256-byte line per XCD slot counter
constexpr int64_t kMaxTasks = int64_t(1) << 30;
// Initial size of a device's pinned staging ring for variable-length tables (the table
// of 16 384 tokens at hidden size 2048 is about 2 MB).
constexpr size_t kStagingBytes = size_t(64) << 20;

// Device memory of dash_attn_bwd_noalloc, for callers that cannot allocate: every device
// the library runs on holds one copy of this array from the loading of the library to
// the end of the process. The first kScratchTableBytes hold schedule tables (and, once,
// at device set-up, the topology probe's output), the rest is the call's workspace.
// Host code never uses the array's name as an address: the per-device address comes
// from hipGetSymbolAddress at set-up (DeviceState::scratch).
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr size_t kScratchTableBytes = size_t(8) << 20;
__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];
// The first kStatusSlots ints of the array (inside its table part) are the per-stream
// status slots of dash_last_kernel_error: each backward call's last kernel copies the
// call's error word into its stream's slot. Tables start at kScratchTablesStart.
constexpr int kStatusSlots = 4096;
constexpr size_t kScratchTablesStart = size_t(64) << 10;
static_assert(kStatusSlots * sizeof(int) <= kScratchTablesStart, "status slots fit before the tables");

int tile_for(int N) { return N < 512 ? 64 : 128; }


int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
  size_t dqacc = 0, neg_delta = 0, nlse2 = 0, sem = 0, ctr = 0, err = 0, total = 0;
  int sem_stride = 0;
  int row_stride = 0;  // rows per head of -D, -LSE*log2(e) and the dQ accumulator: N rounded up to the tile
};

// Per-tile partials (deterministic = 3): one slot of 64 x d floats per (b, h, 64-row step,
// contribution); a head has (tile / 64) x n^2 slots, n (n + 1) / 2 instead of n^2 for the
// causal mask (partial_slot in kernels.h).
size_t partials_bytes(int B, int H, int N, int d, bool causal) {
  const int tile = tile_for(N);
  const int64_t n = cdiv(N, tile);
  const int64_t per_head = (causal ? n * (n + 1) / 2 : n * n) * (tile / 64);
  return align256(size_t(B) * H * per_head * 64 * d * sizeof(float));
}

WsLayout ws_layout(int B, int H, int N, int d, size_t dq_bytes_override = 0) {
  WsLayout L;
  // One semaphore per 64-row Q step and wave (dash::kSemPerStep at most), for every
  // step of the ceil(N / tile) tiles of a head (the last tile's second step may lie past N).
  const int tile = tile_for(N);
  L.sem_stride = static_cast<int>(cdiv(cdiv(N, tile) * (tile / 64) * dash::kSemPerStep, 32) * 32);
  L.row_stride = static_cast<int>(cdiv(N, tile) * tile);
  const size_t dq_bytes =
      dq_bytes_override ? dq_bytes_override : align256(size_t(B) * H * L.row_stride * d * sizeof(float));
  const size_t row_bytes = align256(size_t(B) * H * L.row_stride * sizeof(float));
  const size_t sem_bytes = align256(size_t(B) * H * L.sem_stride * sizeof(int));
  L.dqacc = 0;
  L.neg_delta = L.dqacc + dq_bytes;
  L.nlse2 = L.neg_delta + row_bytes;
  L.sem = L.nlse2 + row_bytes;
  L.ctr = L.sem + sem_bytes;
  L.err = L.ctr + kCtrInts * sizeof(int);  // the call's error word, on a 256-byte line of its own
  L.total = L.err + 256;
  return L;
}

// Checks shared by every entry point; pointers are checked separately.
// A valid stand-in for DASH_SCHED_AUTO while the arguments are checked (the call itself
// resolves AUTO with the cost model below once the device topology is known): shift for
// the full mask, symmetric shift for the causal mask, descending when the tile count is
// odd (symmetric shift is not defined there). Other values are returned unchanged.
int resolve_schedule(int schedule, int N, int mask) {
  if (schedule != DASH_SCHED_AUTO) return schedule;
  if (mask != DASH_MASK_CAUSAL) return DASH_SCHED_SHIFT;
  return cdiv(N, tile_for(N)) % 2 == 0 ? DASH_SCHED_SYM_SHIFT : DASH_SCHED_DESCENDING;
}

// Costs of one task (one KV tile against one Q tile) on MI355X for the hardware-aware
// schedule model (DASH paper, section 3.1 model; section 4.2 local vs remote L2
// segments), in microseconds, measured with the library's kernels:
//  - d = 128, 128-row tiles: full mask, B=8, H=16, N=2048: main kernel at 828 TFLOP/s with the
//    ordered reduction and 960 TFLOP/s with the reduction's memory traffic removed, over
//    256 CUs and 20.97 MFLOP per task: c = 5.6, r_local = 0.9;
//  - d = 64: causal mask, B=4, H=32, N=4096: main kernel 0.962 ms for 264 tasks per CU,
//    split in the same proportion: c = 3.2, r_local = 0.45;
//  - r_remote: dQ chains across XCDs (causal mask, B=1, H=16, N=16384, d=128, symmetric shift)
//    ran at 688 TFLOPS against 861 inside one XCD, 7.8 us instead of 6.2 us per task:
//    r_remote = 0.9 + 1.6 = 2.5, taken for both d (device-scope running sums and flags).
// 64-row tiles (N < 512) do a quarter of the contraction work and half of the dQ
// traffic per task. The same kernel binary runs every schedule (the table is data), so
// the model has no schedule-dependent register term.
dash::CostModel measured_costs(int d, int tile) {
  dash::CostModel m;
  m.c = d == 128 ? 5.6 : 3.2;
  m.r_local = d == 128 ? 0.9 : 0.45;
  m.r_remote = 2.5;
  if (tile == 64) {
    m.c *= 0.25;
    m.r_local *= 0.5;
  }
  return m;
}

// Margin by which naive or descending must beat the shift schedule of the mask in the
// model before AUTO takes it. The model prices every reduction at r_local or r_remote;
// on the GPU a reduction waits for its predecessor's, and a contribution is added during
// the CU's next step, so chains whose contributors follow each other step after step
// (naive and descending: a wavefront over the tile's lanes) lose up to about a task per
// link, while the shift schedules are conflict-free by construction (one contributor per
// dQ tile per time step) and lose nothing. Measured on MI355X: every shape where the
// model put descending within 3 % of symmetric shift ran faster with symmetric shift
// (by 16 % and 43 %), and every shape where it put descending 10 % or more ahead ran
// faster with descending.
constexpr double kShiftMargin = 0.08;

// DASH_SCHED_AUTO: the shift schedule of the mask (shift for the full mask, symmetric
// shift for the causal mask with an even tile count) unless naive or descending has a
// makespan more than kShiftMargin smaller under measured_costs on the tables built for
// this topology and placement; then the smaller of those two (ties to descending).
// Returns a dash_status code on error.
int model_schedule(int B, int H, int Hkv, int N, int d, int mask, int num_xcd, int cus_per_xcd, bool spread) {
  const bool causal = mask == DASH_MASK_CAUSAL;
  const int tile = tile_for(N);
  const int n = static_cast<int>(cdiv(N, tile));
  const int cands[3] = {DASH_SCHED_NAIVE, DASH_SCHED_DESCENDING, causal ? DASH_SCHED_SYM_SHIFT : DASH_SCHED_SHIFT};
  const dash::CostModel m = measured_costs(d, tile);
  int best = -1;
  double best_t = 0.0;
  double shift_t = -1.0;
  for (int sched : cands) {
    if (sched == DASH_SCHED_SYM_SHIFT && n % 2) continue;
    dash::SchedParams sp;
    sp.B = B;
    sp.H = H;
    sp.Hkv = Hkv;
    sp.N = N;
    sp.tile = tile;
    sp.causal = causal;
    sp.kind = static_cast<Sched>(sched);
    sp.num_xcd = num_xcd;
    sp.cus_per_xcd = cus_per_xcd;
    sp.spread = spread;
    dash::Table t;
    std::string err;
    const int s = dash::build_table(sp, &t, &err);
    if (s != 0) return s;
    double span = 0.0;
    if (!dash::table_makespan(t, cus_per_xcd, m, &span)) continue;  // (validated tables never cycle)
    if (sched == DASH_SCHED_SHIFT || sched == DASH_SCHED_SYM_SHIFT) {
      shift_t = span;
      continue;
    }
    if (best < 0 || span <= best_t) {
      best = sched;
      best_t = span;
    }
  }
  if (shift_t >= 0.0 && (best < 0 || best_t >= (1.0 - kShiftMargin) * shift_t))
    return causal ? DASH_SCHED_SYM_SHIFT : DASH_SCHED_SHIFT;
  return best < 0 ? DASH_ERR_UNSUPPORTED : best;
}

// deterministic = 4 (DASH_DET_AUTO): the bitwise-reproducible mode measured faster on
// MI355X for the shape, between the ordered reduction (1) and the two-pass variant (2),
// which take the same workspace. With grouped-query attention of G query heads per KV
// head the ordered reduction has B * Hkv * n lanes (half that for symmetric shift), a
// KV item runs G times the tasks, and in the symmetric shift's phase-2 triangles the
// group's Q, dO and dQ tiles are hot in one XCD's L2 at once; the two-pass variant's dQ
// pass is parallel over query heads. Measured (whole call; N = 2048 .. 8192, d = 64 and
// 128, both masks; heads outermost in the full mask's rows and phase 1): the ordered
// reduction is faster for G <= 2 everywhere (1 - 11 %) and for G = 4 except the causal
// mask at d = 128 and N = 8192 (two-pass 5 % faster there, 6 % slower at N = 2048); the
// two-pass variant is faster for G = 8 everywhere (0.3 - 9 %). 64-row tiles (N < 512)
// keep the ordered reduction.
int resolve_deterministic(int H, int Hkv, int N, int d, int mask, int deterministic) {
  if (deterministic != 4) return deterministic;
  const int G = H / Hkv;
  if (tile_for(N) == 64) return 1;
  if (G >= 8) return 2;
  if (G >= 4 && mask == DASH_MASK_CAUSAL && d == 128 && N >= 4096) return 2;
  return 1;
}

int check_sizes(int B, int H, int Hkv, int N, int d, int mask, int schedule) {
  if (B < 0 || N < 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0) return DASH_ERR_INVALID_ARG;
  if (N > (1 << 22) || int64_t(B) * H > (int64_t(1) << 24)) return DASH_ERR_INVALID_ARG;
  if (mask != DASH_MASK_FULL && mask != DASH_MASK_CAUSAL) return DASH_ERR_INVALID_ARG;
  if (schedule < DASH_SCHED_NAIVE || schedule > DASH_SCHED_SYM_SHIFT) return DASH_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return DASH_ERR_UNSUPPORTED;
  const bool causal = mask == DASH_MASK_CAUSAL;
  if (schedule == DASH_SCHED_SHIFT && causal) return DASH_ERR_UNSUPPORTED;
  if (schedule == DASH_SCHED_SYM_SHIFT && !causal) return DASH_ERR_UNSUPPORTED;
  const int64_t n = cdiv(N, tile_for(N));
  if (schedule == DASH_SCHED_SYM_SHIFT && (n % 2) != 0) return DASH_ERR_UNSUPPORTED;
  const int64_t per_head = causal ? n * (n + 1) / 2 : n * n;
  if (int64_t(B) * H * per_head > kMaxTasks) return DASH_ERR_INVALID_ARG;
  return DASH_OK;
}

// Host image of a device table: worker_begin | items | tasks | step records | batch lengths,
// each part 256-byte aligned.
struct TableImage {
  std::vector<char> bytes;
  size_t it_off = 0, tk_off = 0, st_off = 0, ln_off = 0;
  bool has_lens = false;
  int workers = 0;
  int tile = 0;
  bool xcd_local = true;
};

struct DevTable {
  void* buf = nullptr;  // worker_begin | items | tasks | steps
  const int* worker_begin = nullptr;
  const int4* items = nullptr;
  const int4* tasks = nullptr;
  const int4* steps = nullptr;
  const int* seqlens = nullptr;  // variable-length tables: the batch lengths
  int workers = 0;
  int tile = 0;
  bool xcd_local = true;
};

struct DeviceState {
  bool ready = false;
  int status = DASH_OK;
  int cus = 0;
  int num_xcd = 1;
  int cus_per_xcd = 1;
  long long ticks_per_second = 100000000LL;
  // Status slot (index into the scratch array's first ints) of each stream that has run
  // a backward call; slots are handed out in order and reused round robin past
  // kStatusSlots streams.
  std::map<void*, int> stream_slot;
  int next_slot = 0;
  int* err_host = nullptr;  // pinned word that dash_last_kernel_error copies into (g_err_mu)
  // This device's copy of `scratch` (hipGetSymbolAddress at set-up), and the schedule
  // tables dash_attn_bwd_noalloc has copied into its table part: key -> (offset, image).
  char* scratch = nullptr;
  size_t scratch_tables_used = 0;
  std::map<std::tuple<int, int, int, int, int, int, int, int>, std::pair<size_t, TableImage>> scratch_tables;
  std::map<std::tuple<int, int, int, int, int, int, int, int>, DevTable> tables;
  // Variable-length batches: pinned staging for the stream-ordered table copies into the
  // caller's workspace (allocated at device set-up, grown only for a table larger than it).
  struct Staging {
    char* buf = nullptr;
    size_t cap = 0;
    struct Seg {
      size_t off, size;
      hipEvent_t done;  // recorded on the call's stream after the copy
    };
    std::deque<Seg> inflight;  // in enqueue order
    std::vector<hipEvent_t> idle_events;
  } staging;
};

std::mutex g_mu;
std::mutex g_err_mu;  // the pinned words of dash_last_kernel_error
std::map<int, DeviceState> g_devices;
unsigned long long* g_prof = nullptr;  // profiling builds: device buffer for the phase counters
int g_placement = DASH_PLACEMENT_AGGREGATE;  // CU-group placement of later tables
int g_kernel = DASH_KERNEL_AUTO;  // main-kernel choice of later calls
long long g_wait_timeout_us = 5000000;  // bound of every in-kernel wait (5 s)
// DASH_SCHED_AUTO resolutions, per (B, H, Hkv, N, d, mask, XCDs, CUs per XCD, placement).
std::map<std::tuple<int, int, int, int, int, int, int, int, int>, int> g_auto;
// What DASH_KERNEL_AUTO resolves to where the two-waves-per-SIMD kernel applies: that
// kernel, measured at least as fast as the one-wave kernel on every d = 128 workload.
constexpr bool kPairAuto = true;
#ifdef DASH_REPLAY
float* g_replay = nullptr;              // replay builds: dump of the ordered dQ partials
size_t g_replay_bytes = 0;
#endif

// Measures which XCD each workgroup of a one-per-CU grid lands on. A clean
// round-robin split (every XCD id present with the same count) gives the table
// topology; anything else falls back to one domain spanning all CUs.
int init_device(int dev, DeviceState* st) {
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DASH_ERR_HIP;
  st->cus = prop.multiProcessorCount;
  int rate_khz = 0;
  if (hipDeviceGetAttribute(&rate_khz, hipDeviceAttributeWallClockRate, dev) == hipSuccess && rate_khz > 0)
    st->ticks_per_second = static_cast<long long>(rate_khz) * 1000LL;
  // This device's copy of the scratch array (its address differs per device). Set-up
  // allocates nothing: the probe below writes into the scratch array's table part, which
  // no call uses yet.
  void* scr = nullptr;
  if (hipGetSymbolAddress(&scr, HIP_SYMBOL(scratch)) != hipSuccess || scr == nullptr) return DASH_ERR_HIP;
  st->scratch = static_cast<char*>(scr);
  if (kScratchTablesStart + size_t(st->cus) * sizeof(int) > kScratchTableBytes) return DASH_ERR_UNSUPPORTED;
  int* probe = reinterpret_cast<int*>(st->scratch + kScratchTablesStart);
  hipError_t e = dash::launch_topology_probe(probe, st->cus, nullptr);
  std::vector<int> ids(st->cus, -1);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e == hipSuccess) e = hipMemcpy(ids.data(), probe, sizeof(int) * st->cus, hipMemcpyDeviceToHost);
  if (e == hipErrorCooperativeLaunchTooLarge) return DASH_ERR_NOT_CORESIDENT;
  if (e != hipSuccess) return DASH_ERR_HIP;
  int max_id = -1;
  std::vector<int> count(16, 0);
  bool sane = true;
  for (int x : ids) {
    if (x < 0 || x >= 16) {
      sane = false;
      break;
    }
    count[x]++;
    if (x > max_id) max_id = x;
  }
  st->num_xcd = 1;
  st->cus_per_xcd = st->cus;
  if (sane && max_id >= 1) {
    const int X = max_id + 1;
    bool even = (st->cus % X) == 0;
    for (int x = 0; x < X && even; ++x) even = count[x] == st->cus / X;
    if (even) {
      st->num_xcd = X;
      st->cus_per_xcd = st->cus / X;
    }
  }
  st->ready = true;
  return DASH_OK;
}

int get_device(DeviceState** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DASH_ERR_HIP;
  DeviceState& st = g_devices[dev];
  if (!st.ready) {
    if (st.status != DASH_OK) return st.status;
    const int s = init_device(dev, &st);
    if (s != DASH_OK) {
      st.status = s;
      return s;
    }
  }
  *out = &st;
  return DASH_OK;
}

int upload_table(const dash::Table& t, int H, int tile, const std::vector<int>* lens, DevTable* out);

int get_table(DeviceState* st, int B, int H, int Hkv, int N, bool causal, int schedule, const DevTable** out) {
  const int tile = tile_for(N);
  auto key = std::make_tuple(B, H, Hkv, N, tile, causal ? 1 : 0, schedule, g_placement);
  auto found = st->tables.find(key);
  if (found != st->tables.end()) {
    *out = &found->second;
    return DASH_OK;
  }
  dash::SchedParams sp;
  sp.B = B;
  sp.H = H;
  sp.Hkv = Hkv;
  sp.N = N;
  sp.tile = tile;
  sp.causal = causal;
  sp.kind = static_cast<Sched>(schedule);
  sp.num_xcd = st->num_xcd;
  sp.cus_per_xcd = st->cus_per_xcd;
  sp.spread = g_placement == DASH_PLACEMENT_SPREAD;
  dash::Table t;
  std::string err;
  const int s = dash::build_table(sp, &t, &err);
  if (s != 0) return s;
  DevTable dt;
  const int u = upload_table(t, H, tile, nullptr, &dt);
  if (u != DASH_OK) return u;
  auto ins = st->tables.emplace(key, dt);
  *out = &ins.first->second;
  return DASH_OK;
}

void make_image(const dash::Table& t, int H, int tile, const std::vector<int>* lens, TableImage* img) {
  const size_t wb_bytes = align256(sizeof(int32_t) * t.worker_begin.size());
  const size_t it_bytes = align256(sizeof(dash::Item) * t.items.size());
  const size_t tk_bytes = align256(sizeof(dash::Task) * (t.tasks.size() + 1));
  // The kernel's step stream: one record {b * H + h, first Q row, rank, last} per 64-row
  // step, in task order (each worker's steps are contiguous, across its items), so that a
  // step's bookkeeping is one record read ahead of time. Two zero records follow, for
  // the read-ahead past a worker's last step (a valid head 0, row 0).
  const int subs = tile / 64;
  std::vector<int4> steps;
  steps.reserve(t.tasks.size() * subs + 2);
  for (size_t k = 0; k < t.tasks.size(); ++k) {
    const dash::Task& tk = t.tasks[k];
    const dash::Item& it = t.items[t.task_item[k]];
    for (int sub = 0; sub < subs; ++sub)
      steps.push_back(int4{it.b * H + tk.h, tk.j * tile + sub * 64, tk.rank, tk.last});
  }
  steps.push_back(int4{0, 0, 0, 0});
  steps.push_back(int4{0, 0, 0, 0});
  const size_t st_bytes = align256(sizeof(int4) * steps.size());
  const size_t ln_bytes = lens ? align256(sizeof(int) * lens->size()) : 0;
  img->it_off = wb_bytes;
  img->tk_off = wb_bytes + it_bytes;
  img->st_off = img->tk_off + tk_bytes;
  img->ln_off = img->st_off + st_bytes;
  img->has_lens = lens != nullptr;
  img->bytes.assign(img->ln_off + ln_bytes, 0);
  char* h = img->bytes.data();
  std::memcpy(h, t.worker_begin.data(), sizeof(int32_t) * t.worker_begin.size());
  std::memcpy(h + img->it_off, t.items.data(), sizeof(dash::Item) * t.items.size());
  if (!t.tasks.empty()) std::memcpy(h + img->tk_off, t.tasks.data(), sizeof(dash::Task) * t.tasks.size());
  std::memcpy(h + img->st_off, steps.data(), sizeof(int4) * steps.size());
  if (lens) std::memcpy(h + img->ln_off, lens->data(), sizeof(int) * lens->size());
  img->workers = t.workers;
  img->tile = tile;
  img->xcd_local = t.xcd_local;
}

// The table's device pointers once its image sits at `base` in device memory.
DevTable table_at(const TableImage& img, void* base) {
  DevTable dt;
  char* b = static_cast<char*>(base);
  dt.buf = base;
  dt.worker_begin = reinterpret_cast<const int*>(b);
  dt.items = reinterpret_cast<const int4*>(b + img.it_off);
  dt.tasks = reinterpret_cast<const int4*>(b + img.tk_off);
  dt.steps = reinterpret_cast<const int4*>(b + img.st_off);
  dt.seqlens = img.has_lens ? reinterpret_cast<const int*>(b + img.ln_off) : nullptr;
  dt.workers = img.workers;
  dt.tile = img.tile;
  dt.xcd_local = img.xcd_local;
  return dt;
}

// Device copy of a table in library-owned memory (the per-shape cache; built once).
int upload_table(const dash::Table& t, int H, int tile, const std::vector<int>* lens, DevTable* out) {
  TableImage img;
  make_image(t, H, tile, lens, &img);
  void* buf = nullptr;
  if (hipMalloc(&buf, img.bytes.size()) != hipSuccess) return DASH_ERR_HIP;
  if (hipMemcpy(buf, img.bytes.data(), img.bytes.size(), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipFree(buf);
    return DASH_ERR_HIP;
  }
  *out = table_at(img, buf);
  return DASH_OK;
}

// Variable-length batches: the length at which the cost model prices batch b (its own
// length, raised to 512 when the padded length N uses 128-row tiles, so that the model
// prices the tile the table uses), and whether its tile count is odd (no symmetric shift).
int varlen_model_len(int N, int len) { return tile_for(N) == 128 && len < 512 ? 512 : len; }
bool varlen_odd_tiles(int N, int len) { return cdiv(len, tile_for(N)) % 2 != 0; }

// Workers a variable-length table is built for at most (compute units of the device; an
// MI355X has 256).
constexpr int kMaxWorkers = 1024;

// Bytes of the workspace region that holds a variable-length batch's table: an upper
// bound of the image of any such table for these sizes (every batch at the padded length
// and the full mask: B * H * n^2 tasks, B * Hkv * n items).
size_t varlen_table_bound(int B, int H, int Hkv, int N) {
  const int tile = tile_for(N);
  const int64_t n = cdiv(N, tile);
  const int64_t tasks = int64_t(B) * H * n * n;
  const int64_t items = int64_t(B) * Hkv * n + 1;
  const int64_t steps = tasks * (tile / 64) + 2;
  return align256(sizeof(int32_t) * (kMaxWorkers + 1)) + align256(16 * items) + align256(16 * (tasks + 1)) +
         align256(16 * steps) + align256(sizeof(int) * size_t(B));
}

// Host images of variable-length tables, most recently used first (bounded; an image is
// rebuilt when its lengths come back after eviction).
constexpr size_t kVarlenImages = 64;
std::list<std::pair<std::vector<int>, TableImage>> g_varlen_images;

int varlen_image(DeviceState* st, int B, int H, int Hkv, int N, bool causal, const std::vector<int>& lens,
                 const std::vector<int>& scheds, const TableImage** out) {
  std::vector<int> key = {st->num_xcd, st->cus_per_xcd, B, H, Hkv, N, causal ? 1 : 0, g_placement};
  key.insert(key.end(), lens.begin(), lens.end());
  key.insert(key.end(), scheds.begin(), scheds.end());
  for (auto it = g_varlen_images.begin(); it != g_varlen_images.end(); ++it) {
    if (it->first == key) {
      g_varlen_images.splice(g_varlen_images.begin(), g_varlen_images, it);
      *out = &g_varlen_images.front().second;
      return DASH_OK;
    }
  }
  dash::SchedParams sp;
  sp.B = B;
  sp.H = H;
  sp.Hkv = Hkv;
  sp.N = N;
  sp.tile = tile_for(N);
  sp.causal = causal;
  sp.num_xcd = st->num_xcd;
  sp.cus_per_xcd = st->cus_per_xcd;
  sp.spread = g_placement == DASH_PLACEMENT_SPREAD;
  std::vector<Sched> kinds;
  for (int x : scheds) kinds.push_back(static_cast<Sched>(x));
  dash::Table t;
  std::string err;
  const int s = dash::build_table_varlen(sp, lens, kinds, &t, &err);
  if (s != 0) return s < 0 ? DASH_ERR_INVALID_ARG : s;
  if (t.workers > kMaxWorkers) return DASH_ERR_UNSUPPORTED;
  g_varlen_images.emplace_front(key, TableImage());
  make_image(t, H, sp.tile, &lens, &g_varlen_images.front().second);
  if (g_varlen_images.size() > kVarlenImages) g_varlen_images.pop_back();
  *out = &g_varlen_images.front().second;
  return DASH_OK;
}

// Copies `img` to `dst` (device memory) on `stream` through the device's pinned staging
// ring: the image goes into a free part of the ring and an asynchronous copy, ordered on
// the stream, moves it; an event marks the part free again once the copy has run. The
// host waits only when the ring holds no free part of this size (copies of earlier calls
// still queued behind other work). Caller holds g_mu.
int stage_table(DeviceState* st, const TableImage& img, void* dst, hipStream_t stream) {
  auto& R = st->staging;
  const size_t size = align256(img.bytes.size());
  auto retire_front = [&](bool wait) -> bool {
    if (R.inflight.empty()) return false;
    const hipError_t q = wait ? hipEventSynchronize(R.inflight.front().done) : hipEventQuery(R.inflight.front().done);
    if (q != hipSuccess) return false;
    R.idle_events.push_back(R.inflight.front().done);
    R.inflight.pop_front();
    return true;
  };
  while (retire_front(false)) {
  }
  if (R.buf == nullptr) {
    // First variable-length call on this device.
    if (hipHostMalloc(reinterpret_cast<void**>(&R.buf), kStagingBytes, hipHostMallocDefault) != hipSuccess)
      return DASH_ERR_HIP;
    R.cap = kStagingBytes;
  }
  if (size > R.cap) {
    // A table larger than the ring: wait for the copies in flight and grow it.
    while (retire_front(true)) {
    }
    if (!R.inflight.empty()) return DASH_ERR_HIP;
    if (R.buf) (void)hipHostFree(R.buf);
    R.buf = nullptr;
    R.cap = 0;
    if (hipHostMalloc(reinterpret_cast<void**>(&R.buf), size, hipHostMallocDefault) != hipSuccess) return DASH_ERR_HIP;
    R.cap = size;
  }
  // The parts in flight occupy the ring from the oldest part's offset onward, in enqueue
  // order, wrapping to 0 at most once: free space is after the newest part and, while the
  // newest part lies after the oldest, also before the oldest.
  size_t off = 0;
  while (!R.inflight.empty()) {
    const auto& first = R.inflight.front();
    const auto& last = R.inflight.back();
    const size_t end = last.off + last.size;
    if (last.off >= first.off) {
      if (end + size <= R.cap) {
        off = end;
        break;
      }
      if (size <= first.off) {
        off = 0;
        break;
      }
    } else if (end + size <= first.off) {
      off = end;
      break;
    }
    if (!retire_front(true)) return DASH_ERR_HIP;
  }
  std::memcpy(R.buf + off, img.bytes.data(), img.bytes.size());
  hipEvent_t ev = nullptr;
  if (!R.idle_events.empty()) {
    ev = R.idle_events.back();
    R.idle_events.pop_back();
  } else if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess) {
    return DASH_ERR_HIP;
  }
  if (hipMemcpyAsync(dst, R.buf + off, img.bytes.size(), hipMemcpyHostToDevice, stream) != hipSuccess ||
      hipEventRecord(ev, stream) != hipSuccess) {
    R.idle_events.push_back(ev);
    return DASH_ERR_HIP;
  }
  R.inflight.push_back({off, size, ev});
  return DASH_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// dash_attn_bwd_noalloc: the table of this shape in the scratch array's table part,
// copied there on the call's stream the first time the shape comes (the tables of
// earlier shapes are dropped when the part is full). The copy reads pageable host
// memory, which HIP stages before hipMemcpyAsync returns; the image is kept all the same.
// Caller holds g_mu.
int get_table_scratch(DeviceState* st, int B, int H, int Hkv, int N, bool causal, int schedule, hipStream_t stream,
                      DevTable* out) {
  const int tile = tile_for(N);
  const auto key = std::make_tuple(B, H, Hkv, N, tile, causal ? 1 : 0, schedule, g_placement);
  auto found = st->scratch_tables.find(key);
  if (found != st->scratch_tables.end()) {
    *out = table_at(found->second.second, st->scratch + found->second.first);
    return DASH_OK;
  }
  dash::SchedParams sp;
  sp.B = B;
  sp.H = H;
  sp.Hkv = Hkv;
  sp.N = N;
  sp.tile = tile;
  sp.causal = causal;
  sp.kind = static_cast<Sched>(schedule);
  sp.num_xcd = st->num_xcd;
  sp.cus_per_xcd = st->cus_per_xcd;
  sp.spread = g_placement == DASH_PLACEMENT_SPREAD;
  dash::Table t;
  std::string err;
  const int s = dash::build_table(sp, &t, &err);
  if (s != 0) return s;
  TableImage img;
  make_image(t, H, tile, nullptr, &img);
  const size_t size = align256(img.bytes.size());
  if (size > kScratchTableBytes - kScratchTablesStart) return DASH_ERR_WORKSPACE;
  if (st->scratch_tables_used + size > kScratchTableBytes - kScratchTablesStart) {
    st->scratch_tables.clear();
    st->scratch_tables_used = 0;
  }
  const size_t off = kScratchTablesStart + st->scratch_tables_used;
  if (hipMemcpyAsync(st->scratch + off, img.bytes.data(), img.bytes.size(), hipMemcpyHostToDevice, stream) !=
      hipSuccess)
    return DASH_ERR_HIP;
  st->scratch_tables_used += size;
  auto ins = st->scratch_tables.emplace(key, std::make_pair(off, std::move(img)));
  *out = table_at(ins.first->second.second, st->scratch + off);
  return DASH_OK;
}

// noalloc: the workspace and the table are the device's scratch array (the caller passes
// no workspace); nothing is allocated.
int run_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse, void* dq,
            void* dk, void* dv, int B, int H, int Hkv, int N, int d, float scale, int mask, int schedule,
            int deterministic, void* workspace, size_t workspace_bytes, void* stream_ptr, void* ev_start,
            void* ev_stop, const int* seqlens = nullptr, bool noalloc = false) {
  const int requested = schedule;
  schedule = resolve_schedule(schedule, N, mask);
  int s = check_sizes(B, H, Hkv, N, d, mask, schedule);
  if (s != DASH_OK) return s;
  if (deterministic < 0 || deterministic > 4) return DASH_ERR_INVALID_ARG;
  deterministic = resolve_deterministic(H, Hkv, N, d, mask, deterministic);
  if (deterministic == 3 && seqlens) return DASH_ERR_UNSUPPORTED;  // per-tile partials: one length
  // Variable-length batches: lengths in [1, N].
  std::vector<int> lens, scheds;
  if (seqlens && B > 0 && N > 0) {
    for (int b = 0; b < B; ++b) {
      if (seqlens[b] < 1 || seqlens[b] > N) return DASH_ERR_INVALID_ARG;
      lens.push_back(seqlens[b]);
    }
    for (int b = 0; b < B; ++b) {
      int sb = requested;
      if (sb != DASH_SCHED_AUTO) {
        const int c = check_sizes(1, H, Hkv, varlen_model_len(N, lens[b]), d, mask, sb);
        if (c != DASH_OK) return c;
        if (sb == DASH_SCHED_SYM_SHIFT && varlen_odd_tiles(N, lens[b])) return DASH_ERR_UNSUPPORTED;
      }
      scheds.push_back(sb);
    }
  }
  if (!(scale > 0.f) || !std::isfinite(scale)) return DASH_ERR_INVALID_ARG;
  if (B == 0 || N == 0) return DASH_OK;
  const void* ptrs[] = {q, k, v, o, dO, dq, dk, dv};
  for (const void* ptr : ptrs)
    if (ptr == nullptr || !aligned(ptr, 16)) return DASH_ERR_INVALID_ARG;
  if (lse == nullptr || !aligned(lse, 4)) return DASH_ERR_INVALID_ARG;
  if (noalloc) {
    if (seqlens || deterministic == 3) return DASH_ERR_UNSUPPORTED;
    workspace_bytes = kScratchBytes - kScratchTableBytes;
  } else if (workspace == nullptr || !aligned(workspace, 256)) {
    return DASH_ERR_INVALID_ARG;
  }
  const WsLayout L = deterministic == 3 ? ws_layout(B, H, N, d, partials_bytes(B, H, N, d, mask == DASH_MASK_CAUSAL))
                                        : ws_layout(B, H, N, d);
  // Variable-length batches: the call's table goes into the workspace after the base part.
  const size_t table_bytes = seqlens ? varlen_table_bound(B, H, Hkv, N) : 0;
  if (workspace_bytes < L.total + table_bytes) return DASH_ERR_WORKSPACE;

  hipStream_t stream = static_cast<hipStream_t>(stream_ptr);
  const bool causal = mask == DASH_MASK_CAUSAL;
  DeviceState* st = nullptr;
  const DevTable* tab = nullptr;
  DevTable varlen_tab;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    s = get_device(&st);
    if (s != DASH_OK) return s;
    if (noalloc) workspace = st->scratch + kScratchTableBytes;
    if (requested == DASH_SCHED_AUTO) {
      const auto key = std::make_tuple(B, H, Hkv, N, d, mask, st->num_xcd, st->cus_per_xcd, g_placement);
      auto it = g_auto.find(key);
      if (it == g_auto.end()) {
        const int r = model_schedule(B, H, Hkv, N, d, mask, st->num_xcd, st->cus_per_xcd,
                                     g_placement == DASH_PLACEMENT_SPREAD);
        if (r < 0) return r;
        it = g_auto.emplace(key, r).first;
      }
      schedule = it->second;
    }
    if (seqlens) {
      // AUTO per batch: the model's choice at the batch's own length (cached like AUTO).
      for (int b = 0; b < B; ++b) {
        if (scheds[b] != DASH_SCHED_AUTO) continue;
        const int nb = varlen_model_len(N, lens[b]);
        const auto key = std::make_tuple(1, H, Hkv, nb, d, mask, st->num_xcd, st->cus_per_xcd, g_placement);
        auto it = g_auto.find(key);
        if (it == g_auto.end()) {
          const int r = model_schedule(1, H, Hkv, nb, d, mask, st->num_xcd, st->cus_per_xcd,
                                       g_placement == DASH_PLACEMENT_SPREAD);
          if (r < 0) return r;
          it = g_auto.emplace(key, r).first;
        }
        scheds[b] = it->second;
        if (scheds[b] == DASH_SCHED_SYM_SHIFT && varlen_odd_tiles(N, lens[b])) scheds[b] = DASH_SCHED_DESCENDING;
      }
      const TableImage* img = nullptr;
      s = varlen_image(st, B, H, Hkv, N, causal, lens, scheds, &img);
      if (s != DASH_OK) return s;
      if (img->bytes.size() > table_bytes) return DASH_ERR_WORKSPACE;  // (the bound holds for every table)
      void* dst = static_cast<char*>(workspace) + L.total;
      s = stage_table(st, *img, dst, stream);
      if (s != DASH_OK) return s;
      varlen_tab = table_at(*img, dst);
      tab = &varlen_tab;
    } else if (noalloc) {
      s = get_table_scratch(st, B, H, Hkv, N, causal, schedule, stream, &varlen_tab);
      tab = &varlen_tab;
    } else {
      s = get_table(st, B, H, Hkv, N, causal, schedule, &tab);
    }
    if (s != DASH_OK) return s;
  }
  char* ws = static_cast<char*>(workspace);
  float* dqacc = reinterpret_cast<float*>(ws + L.dqacc);
  float* neg_delta = reinterpret_cast<float*>(ws + L.neg_delta);
  float* nlse2 = reinterpret_cast<float*>(ws + L.nlse2);
  int* sem = reinterpret_cast<int*>(ws + L.sem);
  int* ctr = reinterpret_cast<int*>(ws + L.ctr);
  int* err = reinterpret_cast<int*>(ws + L.err);
  dash::StatusCopy status;
  status.err_in = err;

  dash::PreParams pp;
  pp.o = static_cast<const __bf16*>(o);
  pp.dO = static_cast<const __bf16*>(dO);
  pp.lse = lse;
  pp.neg_delta = neg_delta;
  pp.nlse2 = nlse2;
  pp.rows = int64_t(B) * H * N;
  pp.N = N;
  pp.row_stride = L.row_stride;
  pp.sem = sem;
  pp.sem_count = int64_t(B) * H * L.sem_stride;
  pp.ctr = ctr;
  pp.ctr_count = kCtrInts;
  pp.err = err;
  pp.seqlens = tab->seqlens;
  pp.H = H;
  pp.dqacc_zero = deterministic == 0 ? dqacc : nullptr;
  pp.zero_count = int64_t(B) * H * L.row_stride * d;
  const int64_t pre_threads = pp.rows * (d / 8);
  const int pre_grid = static_cast<int>(std::min<int64_t>(std::max<int64_t>(cdiv(pre_threads, 256), 1), 4096));
  if (dash::launch_preprocess(pp, d, pre_grid, stream) != hipSuccess) return DASH_ERR_HIP;

  dash::BwdParams bp;
  bp.q = static_cast<const __bf16*>(q);
  bp.k = static_cast<const __bf16*>(k);
  bp.v = static_cast<const __bf16*>(v);
  bp.dO = static_cast<const __bf16*>(dO);
  bp.nlse2 = nlse2;
  bp.neg_delta = neg_delta;
  bp.dk = static_cast<__bf16*>(dk);
  bp.dv = static_cast<__bf16*>(dv);
  bp.dqacc = dqacc;
  bp.dq = nullptr;  // set below when the two-waves kernel writes dQ itself
  bp.sem = sem;
  bp.ctr = ctr;
  bp.err = err;
  bp.worker_begin = tab->worker_begin;
  bp.items = tab->items;
  bp.tasks = tab->tasks;
  bp.steps = tab->steps;
  bp.B = B;
  bp.H = H;
  bp.Hkv = Hkv;
  bp.N = N;
  bp.sem_stride = L.sem_stride;
  bp.row_stride = L.row_stride;
  bp.scale = scale;
  bp.scale_log2 = scale * 1.4426950408889634f;
  bp.causal = causal ? 1 : 0;
  bp.deterministic = deterministic;
  bp.xcd_local = (tab->xcd_local && st->num_xcd > 1) ? 1 : 0;
  bp.num_xcd = st->num_xcd;
  bp.cus_per_xcd = st->cus_per_xcd;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    // ticks = ticks/s * us / 1e6, without overflow for any accepted timeout
    bp.timeout_ticks = st->ticks_per_second / 1000 * g_wait_timeout_us / 1000;
    auto slot = st->stream_slot.find(stream_ptr);
    if (slot == st->stream_slot.end()) {
      slot = st->stream_slot.emplace(stream_ptr, st->next_slot).first;
      st->next_slot = (st->next_slot + 1) % kStatusSlots;
    }
    status.status_out = reinterpret_cast<int*>(st->scratch) + slot->second;
  }
  bp.prof = g_prof;
  bp.replay = nullptr;
  bp.replay_ranks = 0;
  bp.seqlens = tab->seqlens;
#ifdef DASH_REPLAY
  if (g_replay && deterministic) {
    const int tile = tile_for(N);
    const int ranks = static_cast<int>(cdiv(N, tile));
    const size_t need = size_t(B) * H * (L.row_stride / 64) * (2 * (d / 32)) * ranks * 1024 * sizeof(float);
    if (g_replay_bytes < need) return DASH_ERR_WORKSPACE;
    bp.replay = g_replay;
    bp.replay_ranks = ranks;
  }
#endif
  if (ev_start && hipEventRecord(static_cast<hipEvent_t>(ev_start), stream) != hipSuccess) return DASH_ERR_HIP;
  // The two-waves-per-SIMD kernel covers 128-row tiles with the ordered reduction
  // inside one XCD and the atomic variant; everything else runs on the
  // one-wave-per-SIMD kernel.
  int kernel;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    kernel = g_kernel;
  }
  // (The per-tile partials have no chains, so any placement suits the two-waves kernel.)
  const bool pair_ok = tab->tile == 128 && deterministic != 2 &&
                       (deterministic == 0 || deterministic == 3 || bp.xcd_local || st->num_xcd == 1);
  const bool use_pair = pair_ok && (kernel == DASH_KERNEL_TWO_WAVES_PER_SIMD || (kernel == DASH_KERNEL_AUTO && kPairAuto));
  // The ordered reduction in the two-waves kernel with the full mask: the last contributor
  // of every dQ block writes bf16 dQ itself (no cast kernel, and no final fp32 sum in the
  // workspace). With the full mask every last contribution falls on an item's last task,
  // which all CUs reach together; under the causal schedules they are spread over the
  // run, and the extra work on those steps holds up the chains waiting behind them
  // (measured: full mask d = 128 whole call 2.5 % faster, causal d = 128 N = 16384 2 %
  // slower), so the causal calls keep the cast kernel.
  const bool fused_dq = use_pair && deterministic == 1 && !causal;
  if (fused_dq) bp.dq = static_cast<__bf16*>(dq);
  hipError_t e = !use_pair ? dash::launch_main(bp, d, tab->tile / 32, tab->workers, stream)
                 : d == 128 ? dash::launch_pair_d128(bp, tab->workers, stream)
                            : dash::launch_pair_d64(bp, tab->workers, stream);
  if (e == hipErrorCooperativeLaunchTooLarge) return DASH_ERR_NOT_CORESIDENT;
  if (e != hipSuccess) return DASH_ERR_HIP;
  if (ev_stop && hipEventRecord(static_cast<hipEvent_t>(ev_stop), stream) != hipSuccess) return DASH_ERR_HIP;
  hipError_t ec;
  if (deterministic == 2) {
    dash::DqParams dp;
    dp.q = static_cast<const __bf16*>(q);
    dp.k = static_cast<const __bf16*>(k);
    dp.v = static_cast<const __bf16*>(v);
    dp.dO = static_cast<const __bf16*>(dO);
    dp.nlse2 = nlse2;
    dp.neg_delta = neg_delta;
    dp.dq = static_cast<__bf16*>(dq);
    dp.seqlens = tab->seqlens;
    dp.B = B;
    dp.H = H;
    dp.Hkv = Hkv;
    dp.N = N;
    dp.row_stride = L.row_stride;
    dp.n_qt = static_cast<int>(cdiv(N, 128));
    dp.causal = causal ? 1 : 0;
    dp.scale = scale;
    dp.scale_log2 = scale * 1.4426950408889634f;
    dp.err_in = status.err_in;
    dp.status_out = status.status_out;
    ec = dash::launch_dq_pass(dp, d, stream);
  } else if (deterministic == 3) {
    ec = dash::launch_dq_consolidate(dqacc, dq, int64_t(B) * H, N, L.row_stride, tab->tile, d, causal ? 1 : 0, scale,
                                     status, stream);
  } else if (fused_dq) {
    ec = dash::launch_status_copy(status, stream);
  } else if (deterministic == 1) {
    ec = dash::launch_dq_cast_blocks(dqacc, dq, int64_t(B) * H, N, L.row_stride, d, scale, status, stream,
                                     tab->seqlens, H);
  } else {
    ec = dash::launch_dq_cast(dqacc, dq, int64_t(B) * H, N, L.row_stride, d, scale, status, stream, tab->seqlens, H);
  }
  if (ec != hipSuccess) return DASH_ERR_HIP;
  return DASH_OK;
}

}  // namespace

extern "C" {

size_t dash_attn_bwd_workspace_size(int B, int H, int Hkv, int N, int d) {
  if (B < 0 || N < 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0 || (d != 64 && d != 128)) return 0;
  if (N > (1 << 22) || int64_t(B) * H > (int64_t(1) << 24)) return 0;
  return ws_layout(B, H, N, d).total;
}

size_t dash_attn_bwd_partials_workspace_size(int B, int H, int Hkv, int N, int d, int mask) {
  if (dash_attn_bwd_workspace_size(B, H, Hkv, N, d) == 0) return 0;
  if (mask != DASH_MASK_FULL && mask != DASH_MASK_CAUSAL) return 0;
  return ws_layout(B, H, N, d, partials_bytes(B, H, N, d, mask == DASH_MASK_CAUSAL)).total;
}

size_t dash_attn_bwd_varlen_workspace_size(int B, int H, int Hkv, int N, int d) {
  const size_t base = dash_attn_bwd_workspace_size(B, H, Hkv, N, d);
  if (base == 0) return 0;
  return base + varlen_table_bound(B, H, Hkv, N);
}

int dash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv, int N,
                  int d, float softmax_scale, int mask, void* stream) {
  if (B < 0 || N < 0 || H <= 0 || Hkv <= 0 || H % Hkv != 0) return DASH_ERR_INVALID_ARG;
  if (N > (1 << 22) || int64_t(B) * H > (int64_t(1) << 24)) return DASH_ERR_INVALID_ARG;
  if (mask != DASH_MASK_FULL && mask != DASH_MASK_CAUSAL) return DASH_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return DASH_ERR_UNSUPPORTED;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return DASH_ERR_INVALID_ARG;
  if (B == 0 || N == 0) return DASH_OK;
  const void* ptrs[] = {q, k, v, o};
  for (const void* ptr : ptrs)
    if (ptr == nullptr || !aligned(ptr, 16)) return DASH_ERR_INVALID_ARG;
  if (lse == nullptr || !aligned(lse, 4)) return DASH_ERR_INVALID_ARG;
  const int64_t n_qt = cdiv(N, 128);
  if (int64_t(B) * H * n_qt > 0x7fffffff) return DASH_ERR_INVALID_ARG;
  dash::FwdParams fp;
  fp.q = static_cast<const __bf16*>(q);
  fp.k = static_cast<const __bf16*>(k);
  fp.v = static_cast<const __bf16*>(v);
  fp.o = static_cast<__bf16*>(o);
  fp.lse = lse;
  fp.B = B;
  fp.H = H;
  fp.Hkv = Hkv;
  fp.N = N;
  fp.n_qt = static_cast<int>(n_qt);
  fp.causal = mask == DASH_MASK_CAUSAL ? 1 : 0;
  fp.scale_log2 = softmax_scale * 1.4426950408889634f;
  if (dash::launch_fwd(fp, d, static_cast<hipStream_t>(stream)) != hipSuccess) return DASH_ERR_HIP;
  return DASH_OK;
}

int dash_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dO, const float* lse,
                  void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d, float softmax_scale, int mask,
                  int schedule, int deterministic, void* workspace, size_t workspace_bytes, void* stream) {
  return run_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, N, d, softmax_scale, mask, schedule, deterministic,
                 workspace, workspace_bytes, stream, nullptr, nullptr);
}

int dash_attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const void* dO,
                         const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                         const int* seqlens, float softmax_scale, int mask, int schedule, int deterministic,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (seqlens == nullptr && B > 0) return DASH_ERR_INVALID_ARG;
  return run_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, N, d, softmax_scale, mask, schedule, deterministic,
                 workspace, workspace_bytes, stream, nullptr, nullptr, seqlens);
}

int dash_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dO,
                          const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                          float softmax_scale, int mask, int schedule, int deterministic, void* stream) {
  return run_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, N, d, softmax_scale, mask, schedule, deterministic,
                 nullptr, 0, stream, nullptr, nullptr, nullptr, true);
}

int dash_attn_bwd_timed(const void* q, const void* k, const void* v, const void* o, const void* dO,
                        const float* lse, void* dq, void* dk, void* dv, int B, int H, int Hkv, int N, int d,
                        float softmax_scale, int mask, int schedule, int deterministic, void* workspace,
                        size_t workspace_bytes, void* stream, void* main_start, void* main_stop) {
  return run_bwd(q, k, v, o, dO, lse, dq, dk, dv, B, H, Hkv, N, d, softmax_scale, mask, schedule, deterministic,
                 workspace, workspace_bytes, stream, main_start, main_stop);
}

int dash_last_kernel_error(void* stream) {
  const int* word = nullptr;
  int* host = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DASH_ERR_HIP;
    auto found = g_devices.find(dev);
    if (found == g_devices.end() || !found->second.ready) return DASH_OK;
    auto w = found->second.stream_slot.find(stream);
    if (w == found->second.stream_slot.end()) return DASH_OK;
    word = reinterpret_cast<const int*>(found->second.scratch) + w->second;
    if (found->second.err_host == nullptr &&
        hipHostMalloc(reinterpret_cast<void**>(&found->second.err_host), sizeof(int), hipHostMallocDefault) !=
            hipSuccess)
      return DASH_ERR_HIP;
    host = found->second.err_host;
  }
  // Only this stream is waited for: the word is copied into pinned host memory by a copy
  // ordered after the stream's work (hipMemcpy would run on the null stream, which waits
  // for every blocking stream of the device).
  std::lock_guard<std::mutex> lock(g_err_mu);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(host, word, sizeof(int), hipMemcpyDeviceToHost, s) != hipSuccess) return DASH_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return DASH_ERR_HIP;
  return *host;
}

const char* dash_status_string(int status) {
  switch (status) {
    case DASH_OK: return "ok";
    case DASH_ERR_INVALID_ARG: return "invalid argument";
    case DASH_ERR_UNSUPPORTED: return "unsupported configuration";
    case DASH_ERR_WORKSPACE: return "workspace too small";
    case DASH_ERR_NOT_CORESIDENT: return "persistent grid cannot be co-resident";
    case DASH_ERR_HIP: return "HIP runtime error";
    case DASH_ERR_TIMEOUT: return "ordered-reduction wait timed out";
    case DASH_ERR_PLACEMENT: return "workgroup placement does not match the schedule table";
    default: return "unknown status";
  }
}

int dash_tile_size(int N) { return tile_for(N); }

#ifdef DASH_PROFILE
// Profiling builds only: later calls write per-wave phase cycle counters of the main
// kernel ([CUs][waves][8] uint64, see ProfSlot in kernels.h) into `buf` (device
// memory owned by the caller, at least CUs * 4 * 8 * 8 bytes); null detaches.
int dash_profile_attach(void* buf) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_prof = static_cast<unsigned long long*>(buf);
  return DASH_OK;
}
#endif

#ifdef DASH_REPLAY
// Replay builds only: later deterministic calls dump every dQ partial (see dash_replay.h);
// null detaches.
int dash_replay_attach(void* buf, size_t bytes) {
  std::lock_guard<std::mutex> lock(g_mu);
  g_replay = static_cast<float*>(buf);
  g_replay_bytes = buf ? bytes : 0;
  return DASH_OK;
}
#endif

int dash_set_kernel(int kernel) {
  if (kernel != DASH_KERNEL_AUTO && kernel != DASH_KERNEL_ONE_WAVE_PER_SIMD && kernel != DASH_KERNEL_TWO_WAVES_PER_SIMD)
    return DASH_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_mu);
  g_kernel = kernel;
  return DASH_OK;
}

int dash_set_wait_timeout(long long microseconds) {
  if (microseconds < 0 || microseconds > 3600LL * 1000000LL) return DASH_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_mu);
  g_wait_timeout_us = microseconds;
  return DASH_OK;
}

int dash_set_placement(int placement) {
  if (placement != DASH_PLACEMENT_AGGREGATE && placement != DASH_PLACEMENT_SPREAD) return DASH_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lock(g_mu);
  g_placement = placement;
  return DASH_OK;
}

int dash_schedule_resolve(int B, int H, int Hkv, int N, int d, int mask, int schedule, int num_xcd,
                          int cus_per_xcd) {
  const int requested = schedule;
  schedule = resolve_schedule(schedule, N, mask);
  int s = check_sizes(B, H, Hkv, N, d, mask, schedule);
  if (s != DASH_OK) return s;
  if (num_xcd <= 0 || cus_per_xcd <= 0 || num_xcd > 64 || cus_per_xcd > 4096) return DASH_ERR_INVALID_ARG;
  if (requested != DASH_SCHED_AUTO) return schedule;
  bool spread;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    spread = g_placement == DASH_PLACEMENT_SPREAD;
  }
  return model_schedule(B, H, Hkv, N, d, mask, num_xcd, cus_per_xcd, spread);
}

int dash_deterministic_resolve(int B, int H, int Hkv, int N, int d, int mask, int deterministic) {
  const int s = check_sizes(B, H, Hkv, N, d, mask, resolve_schedule(DASH_SCHED_AUTO, N, mask));
  if (s != DASH_OK) return s;
  if (deterministic < 0 || deterministic > 4) return DASH_ERR_INVALID_ARG;
  return resolve_deterministic(H, Hkv, N, d, mask, deterministic);
}

int dash_schedule_makespan(int B, int H, int Hkv, int N, int mask, int schedule, int num_xcd, int cus_per_xcd,
                           double c, double r_local, double r_remote, double* makespan) {
  if (makespan == nullptr || !(c >= 0.0) || !(r_local >= 0.0) || !(r_remote >= 0.0) || !std::isfinite(c) ||
      !std::isfinite(r_local) || !std::isfinite(r_remote))
    return DASH_ERR_INVALID_ARG;
  if (schedule == DASH_SCHED_AUTO) {
    schedule = dash_schedule_resolve(B, H, Hkv, N, 128, mask, schedule, num_xcd, cus_per_xcd);
    if (schedule < 0) return schedule;
  }
  int s = check_sizes(B, H, Hkv, N, 64, mask, schedule);
  if (s != DASH_OK) return s;
  if (num_xcd <= 0 || cus_per_xcd <= 0 || num_xcd > 64 || cus_per_xcd > 4096) return DASH_ERR_INVALID_ARG;
  dash::SchedParams sp;
  sp.B = B;
  sp.H = H;
  sp.Hkv = Hkv;
  sp.N = N;
  sp.tile = tile_for(N);
  sp.causal = mask == DASH_MASK_CAUSAL;
  sp.kind = static_cast<Sched>(schedule);
  sp.num_xcd = num_xcd;
  sp.cus_per_xcd = cus_per_xcd;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    sp.spread = g_placement == DASH_PLACEMENT_SPREAD;
  }
  dash::Table t;
  std::string err;
  s = dash::build_table(sp, &t, &err);
  if (s != 0) return s;
  dash::CostModel m;
  m.c = c;
  m.r_local = r_local;
  m.r_remote = r_remote;
  double span = 0.0;
  if (!dash::table_makespan(t, cus_per_xcd, m, &span)) return DASH_ERR_INVALID_ARG;
  *makespan = span;
  return DASH_OK;
}

int dash_schedule_table_varlen(int B, int H, int Hkv, int N, const int* seqlens, int mask, int schedule, int num_xcd,
                               int cus_per_xcd, int* records, long long capacity, long long* count, int* xcd_local) {
  if (seqlens == nullptr || count == nullptr || capacity < 0 || B <= 0) return DASH_ERR_INVALID_ARG;
  if (num_xcd <= 0 || cus_per_xcd <= 0 || num_xcd > 64 || cus_per_xcd > 4096) return DASH_ERR_INVALID_ARG;
  std::vector<int> lens;
  std::vector<Sched> kinds;
  for (int b = 0; b < B; ++b) {
    if (seqlens[b] < 1 || seqlens[b] > N) return DASH_ERR_INVALID_ARG;
    lens.push_back(seqlens[b]);
    const int nb = varlen_model_len(N, seqlens[b]);
    int sb = schedule;
    if (sb == DASH_SCHED_AUTO) {
      sb = dash_schedule_resolve(1, H, Hkv, nb, 128, mask, sb, num_xcd, cus_per_xcd);
      if (sb < 0) return sb;
      if (sb == DASH_SCHED_SYM_SHIFT && varlen_odd_tiles(N, seqlens[b])) sb = DASH_SCHED_DESCENDING;
    } else {
      const int c = check_sizes(1, H, Hkv, nb, 128, mask, sb);
      if (c != DASH_OK) return c;
      if (sb == DASH_SCHED_SYM_SHIFT && varlen_odd_tiles(N, seqlens[b])) return DASH_ERR_UNSUPPORTED;
    }
    kinds.push_back(static_cast<Sched>(sb));
  }
  dash::SchedParams sp;
  sp.B = B;
  sp.H = H;
  sp.Hkv = Hkv;
  sp.N = N;
  sp.tile = tile_for(N);
  sp.causal = mask == DASH_MASK_CAUSAL;
  sp.num_xcd = num_xcd;
  sp.cus_per_xcd = cus_per_xcd;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    sp.spread = g_placement == DASH_PLACEMENT_SPREAD;
  }
  dash::Table t;
  std::string err;
  int s = dash::build_table_varlen(sp, lens, kinds, &t, &err);
  if (s != 0) return s < 0 ? DASH_ERR_INVALID_ARG : s;
  *count = static_cast<long long>(t.tasks.size());
  if (xcd_local) *xcd_local = t.xcd_local ? 1 : 0;
  if (static_cast<long long>(t.tasks.size()) > capacity) return DASH_ERR_WORKSPACE;
  if (!t.tasks.empty() && records == nullptr) return DASH_ERR_INVALID_ARG;
  for (size_t x = 0; x < t.tasks.size(); ++x) {
    const dash::Item& it = t.items[t.task_item[x]];
    int* r = records + 7 * x;
    r[0] = t.task_worker[x];
    r[1] = it.b;
    r[2] = t.tasks[x].h;
    r[3] = it.g;
    r[4] = it.i;
    r[5] = t.tasks[x].j;
    r[6] = t.tasks[x].rank;
  }
  return DASH_OK;
}

int dash_schedule_table(int B, int H, int Hkv, int N, int mask, int schedule, int num_xcd, int cus_per_xcd,
                        int* records, long long capacity, long long* count, int* xcd_local) {
  if (schedule == DASH_SCHED_AUTO) {
    schedule = dash_schedule_resolve(B, H, Hkv, N, 128, mask, schedule, num_xcd, cus_per_xcd);
    if (schedule < 0) return schedule;
  }
  int s = check_sizes(B, H, Hkv, N, 64, mask, schedule);
  if (s != DASH_OK) return s;
  if (num_xcd <= 0 || cus_per_xcd <= 0 || count == nullptr || capacity < 0) return DASH_ERR_INVALID_ARG;
  dash::SchedParams sp;
  sp.B = B;
  sp.H = H;
  sp.Hkv = Hkv;
  sp.N = N;
  sp.tile = tile_for(N);
  sp.causal = mask == DASH_MASK_CAUSAL;
  sp.kind = static_cast<Sched>(schedule);
  sp.num_xcd = num_xcd;
  sp.cus_per_xcd = cus_per_xcd;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    sp.spread = g_placement == DASH_PLACEMENT_SPREAD;
  }
  dash::Table t;
  std::string err;
  s = dash::build_table(sp, &t, &err);
  if (s != 0) return s;
  *count = static_cast<long long>(t.tasks.size());
  if (xcd_local) *xcd_local = t.xcd_local ? 1 : 0;
  if (static_cast<long long>(t.tasks.size()) > capacity) return DASH_ERR_WORKSPACE;
  if (!t.tasks.empty() && records == nullptr) return DASH_ERR_INVALID_ARG;
  for (size_t x = 0; x < t.tasks.size(); ++x) {
    const dash::Item& it = t.items[t.task_item[x]];
    int* r = records + 7 * x;
    r[0] = t.task_worker[x];
    r[1] = it.b;
    r[2] = t.tasks[x].h;
    r[3] = it.g;
    r[4] = it.i;
    r[5] = t.tasks[x].j;
    r[6] = t.tasks[x].rank;
  }
  return DASH_OK;
}

}  // extern "C"
