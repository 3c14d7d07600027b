// Task list of the persistent tile-DAG Cholesky + inverse-factor kernel.
//
// G (R x R blocks of 64) = L L^T and M = L^-1 are computed by five task
// kinds on 64 x 64 tiles (k = block column / step):
//   DIAG(k)        k >= 1: L_{k,k-1} = A_{k,k-1} M_{k-1,k-1}^T, then
//                  A_kk -= L_{k,k-1} L_{k,k-1}^T, then factor A_kk into L_kk
//                  and M_kk. k = 0: factor A_00.
//   PANEL_L(i,k)   i >= k+2: L_ik = A_ik M_kk^T
//   PANEL_M(k,j)   j < k:    M_kj = -M_kk S_kj
//   UPD_A(i,j,k)   i >= j > k, (i,j) != (k+1,k+1): A_ij -= L_ik L_jk^T
//   UPD_S(i,j,k)   i > k >= j: S_ij += L_ik M_kj   (S_ij lives in M_ij)
// The list is ordered by as-soon-as-possible start time with unit costs
// (DIAG costs more), which is a topological order: every dependency of a
// task precedes it. Workgroups take tasks in list order, so a task only ever
// waits for tasks that have already been taken by running workgroups.
// Pure C++ (no HIP) so the ordering can be checked on the host.
#pragma once

#include <cstdint>
#include <vector>

namespace nq {

enum CholTaskType : int32_t {
  kTaskDiag = 0,
  kTaskPanelL = 1,
  kTaskPanelM = 2,
  kTaskUpdA = 3,
  kTaskUpdS = 4,
};

struct CholTask {
  int32_t type, i, j, k;
};

// Version counters carried by the flags (see chol.hip):
//   fA(i,j): updates applied to A_ij;   fL(i,k): 1 once L_ik is final;
//   fS(i,j): updates applied to S_ij;   fM(i,j): 1 once M_ij is final.
struct CholDep {
  int32_t kind;    // 0 = fA, 1 = fL, 2 = fS, 3 = fM
  int32_t i, j;
  int32_t version; // wait until the counter reaches this (>= 1)
};

// Dependencies of one task (versions >= 1 only; version 0 is the initial state).
std::vector<CholDep> chol_task_deps(const CholTask& t);

// All tasks for R block rows, in issue order.
std::vector<CholTask> build_chol_schedule(int R);

// Device record of one task: its tile coordinates, up to three flags it
// waits for (index into the 4 R x R flag array, kind-major, and the version
// to reach; -1 = none) and up to three flags it sets when done. For DIAG with
// k >= 1, out[0] is L_{k,k-1}, set as soon as that tile is final.
struct CholDevTask {
  int32_t type, i, j, k;
  int32_t dep[3], dver[3];
  int32_t out[3], over[3];
};
std::vector<CholDevTask> build_chol_dev_tasks(int R);

}  // namespace nq
