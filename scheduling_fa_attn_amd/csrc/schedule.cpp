// Schedule-table builder: which CU runs which (KV tile, Q tile, query head) task,
// in which order, and at which place of its dQ tile's reduction order.
//
// Sources: DASH paper (arXiv 2601.21824), section 3 (normalisation of n KV tiles to
// n SMs, refined or aggregated otherwise), 3.2 (the FlashAttention-3 baseline:
// ascending Q tiles, dQ reduced in ascending KV order), 3.3 (descending Q-tile
// iteration), 3.4 (shift scheduling for the full mask, Fig. 6; symmetric shift with
// two-phase folding for the causal mask, Fig. 7).
//
// MI355X placement. The GPU has several L2 domains (XCDs); the L2 of one XCD is not
// coherent with the others. A "group" is the set of CUs that cooperate on the dQ
// tiles of one KV head: L lanes, L = n (naive, descending, shift) or n/2 (symmetric
// shift, one lane per KV-tile pair). A group never straddles an XCD: if L exceeds
// the CUs of one XCD, the group takes the whole XCD and each CU runs several lanes
// one after another (the paper's "aggregate"). KV heads (units of one batch element
// and one KV head) go to groups round-robin; a group runs its units one after
// another. With grouped-query attention the G query heads that read one KV head all
// run in the KV tile's item, so its tasks stay contiguous. Where every lane of a group
// visits the same number of Q tiles in a phase (shift: the whole row; symmetric shift:
// phase 1), the heads are visited outermost within that phase: all lanes then work on
// one query head at a time, which keeps the conflict-free order of each head and keeps
// only that head's Q, dO and dQ tiles hot in the XCD's L2 (measured on MI355X: 18 %
// faster on a full-mask group of 4 query heads at N = 8192). In the triangles of the
// symmetric shift's phase 2, whose lengths differ per lane, the heads stay innermost.
#include "schedule.h"

#include <algorithm>
#include <unordered_map>

#include <algorithm>
#include <numeric>

namespace dash {

namespace {

// Query tiles of KV tile i in ascending order (causal: only j >= i).
std::vector<int> q_tiles(int n, int i, bool causal) {
  std::vector<int> js;
  for (int j = causal ? i : 0; j < n; ++j) js.push_back(j);
  return js;
}

struct ItemBuild {
  int b, g, i;
  std::vector<int> js;  // Q tiles in visiting order
  // Grouped-query attention: the first `outer` Q tiles are visited heads-outer (all of them
  // for the group's first query head, then for the next), the rest heads-inner.
  int outer = 0;
};

}  // namespace

int build_table(const SchedParams& p, Table* out, std::string* err) {
  if (p.B < 0 || p.N < 0 || p.H <= 0 || p.Hkv <= 0 || p.H % p.Hkv != 0 || p.tile <= 0 ||
      p.num_xcd <= 0 || p.cus_per_xcd <= 0) {
    *err = "invalid sizes";
    return -1;
  }
  const int n = tiles_per_head(p.N, p.tile);
  const int G = p.H / p.Hkv;
  if (p.kind == Sched::Shift && p.causal) {
    *err = "shift scheduling is defined for the full mask only";
    return -2;
  }
  if (p.kind == Sched::SymShift && !p.causal) {
    *err = "symmetric shift scheduling is defined for the causal mask only";
    return -2;
  }
  if (p.kind == Sched::SymShift && (n % 2) != 0) {
    *err = "symmetric shift needs an even number of tiles per head";
    return -2;
  }
  const int X = p.num_xcd, S = p.cus_per_xcd;
  Table& t = *out;
  t = Table();
  t.workers = X * S;
  t.n = n;
  t.tile = p.tile;
  t.xcd_local = true;

  std::vector<std::vector<ItemBuild>> lanes(t.workers);
  const int U = p.B * p.Hkv;  // units: (batch, KV head)
  if (U > 0 && n > 0) {
    const int L = (p.kind == Sched::SymShift) ? n / 2 : n;
    // A group that spreads spans `span` whole domains (lane c on domain c / S, CU c % S);
    // otherwise it sits on one domain.
    const int span = (p.spread && L > S && L % S == 0 && X % (L / S) == 0) ? L / S : 1;
    int C, NG;
    if (span > 1) {
      C = L;
      NG = X / span;
    } else if (L <= S) {
      C = L;
      NG = X * (S / C);
    } else {
      C = S;
      NG = X;
    }
    // group gamma -> one domain: XCD gamma % X, CU slots [(gamma / X) * C, + C);
    // spread: domains [gamma * span, + span), lane c on domain gamma * span + c / S.
    auto worker_of = [&](int gamma, int c) {
      if (span > 1) return (gamma * span + c / S) * S + c % S;
      const int xcd = gamma % X;
      const int slot = (gamma / X) * C + c;
      return xcd * S + slot;
    };
    for (int gamma = 0; gamma < NG && gamma < U; ++gamma) {
      std::vector<int64_t> free_at(C, 0);  // descending: unit-cost finish time per lane
      for (int u = gamma; u < U; u += NG) {
        const int b = u / p.Hkv, g = u % p.Hkv;
        switch (p.kind) {
          case Sched::Naive:
            for (int v = 0; v < L; ++v)
              lanes[worker_of(gamma, v % C)].push_back({b, g, v, q_tiles(n, v, p.causal)});
            break;
          case Sched::Descending:
            for (int i = 0; i < n; ++i) {
              std::vector<int> js = q_tiles(n, i, p.causal);
              std::reverse(js.begin(), js.end());
              int best = 0;
              for (int c = 1; c < C; ++c)
                if (free_at[c] < free_at[best]) best = c;
              free_at[best] += static_cast<int64_t>(js.size()) * G;
              lanes[worker_of(gamma, best)].push_back({b, g, i, std::move(js)});
            }
            break;
          case Sched::Shift:
            for (int v = 0; v < L; ++v) {
              std::vector<int> js(n);
              for (int s = 0; s < n; ++s) js[s] = (v + s) % n;
              lanes[worker_of(gamma, v % C)].push_back({b, g, v, std::move(js), n});
            }
            break;
          case Sched::SymShift: {
            const int half = n / 2;
            for (int pr = 0; pr < L; ++pr) {
              const int w = worker_of(gamma, pr % C);
              std::vector<int> first;  // KV tile pr: phase 1 rectangle, then left triangle
              for (int s = 0; s < half; ++s) first.push_back(half + (pr + s) % half);
              for (int j = pr; j < half; ++j) first.push_back(j);
              std::vector<int> second;  // KV tile n-1-pr: right triangle bottom-up
              for (int j = n - 1; j >= n - 1 - pr; --j) second.push_back(j);
              lanes[w].push_back({b, g, pr, std::move(first), half});
              lanes[w].push_back({b, g, n - 1 - pr, std::move(second)});
            }
            break;
          }
        }
      }
    }
  }

  // Flatten in worker order (heads outermost within an item's first `outer` Q tiles,
  // innermost after them).
  t.worker_begin.assign(t.workers + 1, 0);
  struct Pos {
    int worker, pos;
  };
  std::vector<Pos> where;  // per task: worker and position in that worker's list
  for (int w = 0; w < t.workers; ++w) {
    t.worker_begin[w] = static_cast<int32_t>(t.items.size());
    int pos = 0;
    for (const ItemBuild& it : lanes[w]) {
      t.items.push_back({it.b, it.g, it.i, static_cast<int32_t>(t.tasks.size())});
      auto push = [&](int hh, int j) {
        t.tasks.push_back({it.g * G + hh, j, -1, 0});
        t.task_worker.push_back(w);
        t.task_item.push_back(static_cast<int32_t>(t.items.size() - 1));
        where.push_back({w, pos++});
      };
      const int outer = static_cast<int>(it.js.size()) < it.outer ? static_cast<int>(it.js.size()) : it.outer;
      for (int hh = 0; hh < G; ++hh)
        for (int x = 0; x < outer; ++x) push(hh, it.js[x]);
      for (size_t x = outer; x < it.js.size(); ++x)
        for (int hh = 0; hh < G; ++hh) push(hh, it.js[x]);
    }
  }
  t.worker_begin[t.workers] = static_cast<int32_t>(t.items.size());
  t.items.push_back({0, 0, 0, static_cast<int32_t>(t.tasks.size())});

  // Ranks. naive / descending: ascending KV tile ("ordered by CTA index").
  // shift / symmetric shift: ascending timestamp = (position in the lane, lane).
  const bool by_time = (p.kind == Sched::Shift || p.kind == Sched::SymShift);
  const int64_t chains = static_cast<int64_t>(p.B) * p.H * n;
  std::vector<std::vector<int32_t>> members(static_cast<size_t>(chains));
  for (size_t k = 0; k < t.tasks.size(); ++k) {
    const Item& it = t.items[t.task_item[k]];
    const int64_t c = (static_cast<int64_t>(it.b) * p.H + t.tasks[k].h) * n + t.tasks[k].j;
    members[static_cast<size_t>(c)].push_back(static_cast<int32_t>(k));
  }
  for (auto& m : members) {
    if (by_time) {
      std::sort(m.begin(), m.end(), [&](int32_t a, int32_t b) {
        if (where[a].pos != where[b].pos) return where[a].pos < where[b].pos;
        return where[a].worker < where[b].worker;
      });
    } else {
      std::sort(m.begin(), m.end(), [&](int32_t a, int32_t b) {
        return t.items[t.task_item[a]].i < t.items[t.task_item[b]].i;
      });
    }
    const int cnt = static_cast<int>(m.size());
    int xcd0 = -1;
    for (int r = 0; r < cnt; ++r) {
      t.tasks[m[r]].rank = r;
      t.tasks[m[r]].last = (r == cnt - 1) ? 1 : 0;
      const int xcd = t.task_worker[m[r]] / S;
      if (xcd0 < 0) xcd0 = xcd;
      if (xcd != xcd0) t.xcd_local = false;
    }
  }
  return 0;
}

int build_table_varlen(const SchedParams& p, const std::vector<int>& lens, const std::vector<Sched>& kinds,
                       Table* out, std::string* err) {
  if (static_cast<int>(lens.size()) != p.B || static_cast<int>(kinds.size()) != p.B || p.B < 1) {
    *err = "one length and one schedule per batch";
    return -1;
  }
  for (int b = 0; b < p.B; ++b) {
    if (lens[b] < 1 || lens[b] > p.N) {
      *err = "batch length outside [1, N]";
      return -1;
    }
  }
  const int X = p.num_xcd, S = p.cus_per_xcd;
  const int workers = X * S;
  // Up to S batches run side by side: batch b gets a band of width[b] slots in every L2
  // domain (slots off[b] .. off[b] + width[b] - 1), widths in proportion to the batch's
  // tasks (at least one slot); its table is built for that band as its whole device, so
  // its chains stay inside a domain and batches never wait for each other. More batches
  // than slots share the device: each batch's table is built for the whole device and
  // every worker runs its items of batch 0, then of batch 1, and so on, batch b's
  // workers rotated (whole domains and slots within every domain) to even out the task
  // counts. Reduction chains never cross batches, and in both layouts a worker's batches
  // follow one fixed order, so the merged table is as deadlock-free as its parts.
  const bool banded = p.B <= S;
  std::vector<int> width(p.B, S), off(p.B, 0);
  if (banded) {
    std::vector<double> work(p.B);
    double total = 0.0;
    for (int b = 0; b < p.B; ++b) {
      const double n = static_cast<double>(tiles_per_head(lens[b], p.tile));
      work[b] = p.causal ? n * (n + 1) / 2 : n * n;
      total += work[b];
    }
    int used = 0;
    std::vector<std::pair<double, int>> rem;
    for (int b = 0; b < p.B; ++b) {
      const double share = work[b] / total * (S - p.B);  // one slot each, the rest by share
      width[b] = 1 + static_cast<int>(share);
      used += width[b];
      rem.push_back({share - static_cast<int>(share), b});
    }
    std::sort(rem.begin(), rem.end(), [](const std::pair<double, int>& a, const std::pair<double, int>& c) {
      return a.first > c.first || (a.first == c.first && a.second < c.second);
    });
    for (size_t x = 0; used < S && x < rem.size(); ++x, ++used) ++width[rem[x].second];
    for (int b = 1; b < p.B; ++b) off[b] = off[b - 1] + width[b - 1];
  }
  std::vector<Table> parts(p.B);
  for (int b = 0; b < p.B; ++b) {
    SchedParams q = p;
    q.B = 1;
    q.N = lens[b];
    q.kind = kinds[b];
    q.cus_per_xcd = width[b];
    const int s = build_table(q, &parts[b], err);
    if (s != 0) return s;
  }
  // Worker of batch b's table -> device worker: banded, slot s of domain x goes to slot
  // off[b] + s of domain x; shared, a rotation chosen as described above.
  std::vector<std::vector<int>> dev_of(p.B);
  if (banded) {
    for (int b = 0; b < p.B; ++b) {
      dev_of[b].resize(X * width[b]);
      for (int w = 0; w < X * width[b]; ++w) dev_of[b][w] = (w / width[b]) * S + off[b] + w % width[b];
    }
  } else {
    auto rot = [&](int w, int r) { return ((w / S + r / S) % X) * S + (w % S + r % S) % S; };
    std::vector<int64_t> load(workers, 0);
    for (int b = 0; b < p.B; ++b) {
      const Table& q = parts[b];
      std::vector<int64_t> own(workers, 0);
      for (int w = 0; w < workers; ++w) own[w] = q.items[q.worker_begin[w + 1]].t0 - q.items[q.worker_begin[w]].t0;
      int64_t best = -1;
      int best_r = 0;
      for (int r = 0; r < workers; ++r) {
        int64_t mx = 0;
        for (int w = 0; w < workers; ++w) mx = std::max(mx, load[rot(w, r)] + own[w]);
        if (best < 0 || mx < best) {
          best = mx;
          best_r = r;
        }
      }
      dev_of[b].resize(workers);
      for (int w = 0; w < workers; ++w) {
        dev_of[b][w] = rot(w, best_r);
        load[dev_of[b][w]] += own[w];
      }
    }
  }
  // Items of every device worker: its batches in order.
  std::vector<std::vector<std::pair<int, int>>> runs(workers);  // (batch, table worker)
  for (int b = 0; b < p.B; ++b)
    for (int w = 0; w < static_cast<int>(dev_of[b].size()); ++w) runs[dev_of[b][w]].push_back({b, w});
  Table t;
  t.workers = workers;
  t.tile = p.tile;
  t.n = tiles_per_head(p.N, p.tile);
  t.xcd_local = true;
  for (const Table& q : parts) t.xcd_local = t.xcd_local && q.xcd_local;
  t.worker_begin.push_back(0);
  for (int wd = 0; wd < workers; ++wd) {
    std::sort(runs[wd].begin(), runs[wd].end());
    for (const auto& bw : runs[wd]) {
      const Table& q = parts[bw.first];
      const int w = bw.second;
      for (int x = q.worker_begin[w]; x < q.worker_begin[w + 1]; ++x) {
        Item it = q.items[x];
        const int t0 = it.t0, t1 = q.items[x + 1].t0;
        it.b = bw.first;
        it.t0 = static_cast<int32_t>(t.tasks.size());
        t.items.push_back(it);
        for (int k = t0; k < t1; ++k) {
          t.tasks.push_back(q.tasks[k]);
          t.task_worker.push_back(wd);
          t.task_item.push_back(static_cast<int32_t>(t.items.size() - 1));
        }
      }
    }
    t.worker_begin.push_back(static_cast<int32_t>(t.items.size()));
  }
  t.items.push_back(Item{0, 0, 0, static_cast<int32_t>(t.tasks.size())});
  *out = std::move(t);
  return 0;
}

bool table_makespan(const Table& t, int cus_per_xcd, const CostModel& m, double* makespan) {
  const size_t nt = t.tasks.size();
  // Predecessor of every task on its CU and in its dQ tile's reduction order (-1: none).
  std::vector<int64_t> prev_cu(nt, -1), prev_chain(nt, -1);
  std::vector<int64_t> next_cu(nt, -1), next_chain(nt, -1);
  std::vector<int64_t> last_of_worker(t.workers > 0 ? t.workers : 0, -1);
  for (size_t k = 0; k < nt; ++k) {
    const int w = t.task_worker[k];
    if (last_of_worker[w] >= 0) {
      prev_cu[k] = last_of_worker[w];
      next_cu[last_of_worker[w]] = static_cast<int64_t>(k);
    }
    last_of_worker[w] = static_cast<int64_t>(k);
  }
  // Chains: members of dQ tile (b, h, j), placed by rank.
  std::unordered_map<int64_t, std::vector<int64_t>> chains;
  for (size_t k = 0; k < nt; ++k) {
    const Item& it = t.items[t.task_item[k]];
    const int64_t key = (static_cast<int64_t>(it.b) * 65536 + t.tasks[k].h) * (int64_t(1) << 24) + t.tasks[k].j;
    std::vector<int64_t>& v = chains[key];
    const int r = t.tasks[k].rank;
    if (r < 0) return false;
    if (static_cast<size_t>(r) >= v.size()) v.resize(r + 1, -1);
    if (v[r] >= 0) return false;  // two tasks with one rank
    v[r] = static_cast<int64_t>(k);
  }
  for (const auto& kv : chains) {
    const std::vector<int64_t>& v = kv.second;
    for (size_t r = 1; r < v.size(); ++r) {
      if (v[r] < 0 || v[r - 1] < 0) return false;  // a gap in the ranks
      prev_chain[v[r]] = v[r - 1];
      next_chain[v[r - 1]] = v[r];
    }
  }
  // Kahn's order over tasks; per task: compute start = end of the CU's previous
  // reduction, reduction start = max(compute end, end of the chain predecessor's
  // reduction).
  std::vector<int> indeg(nt, 0);
  std::vector<double> c_start(nt, 0.0), r_floor(nt, 0.0), r_end(nt, 0.0);
  std::vector<int64_t> queue;
  queue.reserve(nt);
  for (size_t k = 0; k < nt; ++k) {
    indeg[k] = (prev_cu[k] >= 0) + (prev_chain[k] >= 0);
    if (indeg[k] == 0) queue.push_back(static_cast<int64_t>(k));
  }
  const int S = cus_per_xcd > 0 ? cus_per_xcd : 1;
  double span = 0.0;
  size_t head = 0;
  while (head < queue.size()) {
    const int64_t k = queue[head++];
    const int64_t pc = prev_chain[k];
    const bool remote = pc >= 0 && t.task_worker[pc] / S != t.task_worker[k] / S;
    const double rs = std::max(c_start[k] + m.c, r_floor[k]);
    r_end[k] = rs + (remote ? m.r_remote : m.r_local);
    span = std::max(span, r_end[k]);
    const int64_t nc = next_cu[k];
    if (nc >= 0) {
      c_start[nc] = std::max(c_start[nc], r_end[k]);
      if (--indeg[nc] == 0) queue.push_back(nc);
    }
    const int64_t nr = next_chain[k];
    if (nr >= 0) {
      r_floor[nr] = std::max(r_floor[nr], r_end[k]);
      if (--indeg[nr] == 0) queue.push_back(nr);
    }
  }
  if (queue.size() != nt) return false;
  *makespan = span;
  return true;
}

}  // namespace dash
