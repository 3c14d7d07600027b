// Host construction of the tile-DAG Cholesky schedule (see chol_schedule.h).
#include "chol_schedule.h"

#include <algorithm>
#include <map>
#include <tuple>

namespace nq {

std::vector<CholDep> chol_task_deps(const CholTask& t) {
  std::vector<CholDep> d;
  const int i = t.i, j = t.j, k = t.k;
  switch (t.type) {
    case kTaskDiag:
      if (k >= 1) d.push_back({1, k - 1, k - 1, 1});        // L_{k-1,k-1}, M_{k-1,k-1}
      if (k >= 2) {
        d.push_back({0, k, k, k - 1});                       // A_kk after updates 0..k-2
        d.push_back({0, k, k - 1, k - 1});                   // A_{k,k-1} after updates 0..k-2
      }
      break;
    case kTaskPanelL:
      d.push_back({1, k, k, 1});                             // M_kk
      if (k >= 1) d.push_back({0, i, k, k});                 // A_ik after updates 0..k-1
      break;
    case kTaskPanelM:
      d.push_back({1, k, k, 1});                             // M_kk
      d.push_back({2, k, j, k - j});                         // S_kj complete (k - j >= 1)
      break;
    case kTaskUpdA:
      d.push_back({1, i, k, 1});
      if (j != i) d.push_back({1, j, k, 1});
      if (k >= 1) d.push_back({0, i, j, k});
      break;
    case kTaskUpdS:
      d.push_back({1, i, k, 1});
      d.push_back({3, k, j, 1});
      if (k - j >= 1) d.push_back({2, i, j, k - j});
      break;
  }
  return d;
}

std::vector<CholTask> build_chol_schedule(int R) {
  std::vector<CholTask> tasks;
  for (int k = 0; k < R; ++k) {
    tasks.push_back({kTaskDiag, k, k, k});
    for (int i = k + 2; i < R; ++i) tasks.push_back({kTaskPanelL, i, k, k});
    for (int j = 0; j < k; ++j) tasks.push_back({kTaskPanelM, k, j, k});
    for (int i = k + 1; i < R; ++i)
      for (int j = k + 1; j <= i; ++j)
        if (!(i == k + 1 && j == k + 1)) tasks.push_back({kTaskUpdA, i, j, k});
    for (int i = k + 1; i < R; ++i)
      for (int j = 0; j <= k; ++j) tasks.push_back({kTaskUpdS, i, j, k});
  }
  // Which task produces each (counter, tile, version).
  std::map<std::tuple<int, int, int, int>, size_t> producer;
  for (size_t n = 0; n < tasks.size(); ++n) {
    const CholTask& t = tasks[n];
    switch (t.type) {
      case kTaskDiag:
        producer[{1, t.k, t.k, 1}] = n;
        producer[{3, t.k, t.k, 1}] = n;
        if (t.k >= 1) producer[{1, t.k, t.k - 1, 1}] = n;
        break;
      case kTaskPanelL: producer[{1, t.i, t.k, 1}] = n; break;
      case kTaskPanelM: producer[{3, t.k, t.j, 1}] = n; break;
      case kTaskUpdA: producer[{0, t.i, t.j, t.k + 1}] = n; break;
      case kTaskUpdS: producer[{2, t.i, t.j, t.k - t.j + 1}] = n; break;
    }
  }
  // As-soon-as-possible start times; the creation order above is already
  // topological, so one forward pass suffices.
  std::vector<double> start(tasks.size(), 0.0), finish(tasks.size(), 0.0);
  for (size_t n = 0; n < tasks.size(); ++n) {
    double s0 = 0.0;
    for (const CholDep& d : chol_task_deps(tasks[n])) {
      // a counter at version v was produced by the task that wrote version v
      auto it = producer.find({d.kind, d.i, d.j, d.version});
      if (it != producer.end()) s0 = std::max(s0, finish[it->second]);
    }
    start[n] = s0;
    const double cost = tasks[n].type == kTaskDiag ? (tasks[n].k ? 8.0 : 5.0) : 1.0;
    finish[n] = s0 + cost;
  }
  std::vector<size_t> order(tasks.size());
  for (size_t n = 0; n < order.size(); ++n) order[n] = n;
  std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) {
    if (start[a] != start[b]) return start[a] < start[b];
    return tasks[a].type < tasks[b].type;
  });
  std::vector<CholTask> out;
  out.reserve(tasks.size());
  for (size_t n : order) out.push_back(tasks[n]);
  return out;
}

std::vector<CholDevTask> build_chol_dev_tasks(int R) {
  const auto idx = [R](int kind, int i, int j) { return (kind * R + i) * R + j; };
  std::vector<CholDevTask> out;
  for (const CholTask& t : build_chol_schedule(R)) {
    CholDevTask d{};
    d.type = t.type; d.i = t.i; d.j = t.j; d.k = t.k;
    for (int q = 0; q < 3; ++q) d.dep[q] = d.out[q] = -1, d.dver[q] = d.over[q] = 0;
    const auto deps = chol_task_deps(t);
    for (size_t q = 0; q < deps.size() && q < 3; ++q) {
      d.dep[q] = idx(deps[q].kind, deps[q].i, deps[q].j);
      d.dver[q] = deps[q].version;
    }
    int no = 0;
    auto put = [&](int kind, int i, int j, int v) {
      d.out[no] = idx(kind, i, j);
      d.over[no] = v;
      ++no;
    };
    switch (t.type) {
      case kTaskDiag:
        if (t.k >= 1) put(1, t.k, t.k - 1, 1);
        put(1, t.k, t.k, 1);
        put(3, t.k, t.k, 1);
        break;
      case kTaskPanelL: put(1, t.i, t.k, 1); break;
      case kTaskPanelM: put(3, t.k, t.j, 1); break;
      case kTaskUpdA: put(0, t.i, t.j, t.k + 1); break;
      case kTaskUpdS: put(2, t.i, t.j, t.k - t.j + 1); break;
    }
    out.push_back(d);
  }
  return out;
}

}  // namespace nq
