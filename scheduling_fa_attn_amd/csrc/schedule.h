// Tile-to-CU schedule tables for the deterministic attention backward.
//
// DASH paper (arXiv 2601.21824), section 3: n KV tiles per head, each KV tile's
// tasks (one per Q tile, and per query head of a grouped-query head group) run
// back to back on one CU; the dQ tile of (batch, query head, Q tile) receives one
// partial sum per contributing KV tile, in an order fixed by the schedule.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace dash {

enum class Sched : int { Naive = 0, Descending = 1, Shift = 2, SymShift = 3 };

struct SchedParams {
  int B = 0, H = 0, Hkv = 0, N = 0;
  int tile = 128;      // KV / Q tile edge in rows
  bool causal = false;
  Sched kind = Sched::Naive;
  int num_xcd = 1;     // L2 domains
  int cus_per_xcd = 1; // compute units per L2 domain
  // Groups with more lanes than one L2 domain has CUs: false = aggregate them on one
  // domain (a CU runs several lanes one after another); true = spread them over as many
  // domains as they need, one lane per CU (the paper's n-SM layout; dQ chains then cross
  // L2 domains).
  bool spread = false;
};

// One task: query head h, Q tile j, place `rank` in dQ tile (b, h, j)'s reduction
// order; `last` = 1 when rank is the final place (that task passes no turn on).
struct Task {
  int32_t h, j, rank, last;
};

// One KV item: batch b, KV head g, KV tile i; its tasks are tasks[t0, next item's t0).
struct Item {
  int32_t b, g, i, t0;
};

struct Table {
  int workers = 0;                  // num_xcd * cus_per_xcd
  int n = 0;                        // tiles per head
  int tile = 0;
  bool xcd_local = true;            // every dQ tile's contributors share one L2 domain
  std::vector<int32_t> worker_begin;  // workers + 1 entries into items
  std::vector<Item> items;            // items.size() = real items + 1 sentinel (t0 = tasks.size())
  std::vector<Task> tasks;
  std::vector<int32_t> task_worker;   // worker of each task (for export)
  std::vector<int32_t> task_item;     // item of each task (for export)
};

// Number of tiles per head for sequence length N and tile edge `tile`.
inline int tiles_per_head(int N, int tile) { return (N + tile - 1) / tile; }

// Builds the table. Returns 0 on success, or a dash_status code with a message in *err.
int build_table(const SchedParams& p, Table* out, std::string* err);

// Variable-length batches: batch b has lens[b] rows (1 <= lens[b] <= p.N) and runs
// schedule kinds[b]. Each batch's table is built as for B = 1 at its own length on the
// whole topology, and every worker runs its items of batch 0, then of batch 1, and so on.
// The reduction chains of different batches never meet, and a worker's batches follow
// each other in one order on every worker, so the merged table is as deadlock-free as
// its parts. Returns 0 or a dash_status code with a message in *err.
int build_table_varlen(const SchedParams& p, const std::vector<int>& lens, const std::vector<Sched>& kinds,
                       Table* out, std::string* err);

// Cost model of a table (DASH paper, section 3.1, "Graph Construction"): every task is
// a compute edge c followed by a reduction edge r on its CU; a CU runs its tasks back
// to back; the reductions into one dQ tile follow each other in rank order (zero-weight
// edge from the end of one to the start of the next). Hardware-aware refinement
// (section 4.2: synchronisation through the local L2 segment is cheaper than through a
// remote one; on MI355X the L2 domains are the XCDs): a reduction whose predecessor in
// its dQ tile's order ran on another L2 domain costs r_remote instead of r_local. The
// first reduction of a tile costs r_local.
struct CostModel {
  double c = 1.0;
  double r_local = 0.0;
  double r_remote = 0.0;
};

// Longest path (makespan) of the table's DAG under `m`, with the CU of worker w on L2
// domain w / cus_per_xcd. Returns false if the DAG has a cycle (the table would
// deadlock), true otherwise.
bool table_makespan(const Table& t, int cus_per_xcd, const CostModel& m, double* makespan);

}  // namespace dash
