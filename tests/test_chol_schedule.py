"""Host-logic checks of the tile-DAG Cholesky schedule (no GPU).

The C++ schedule builder is compiled with g++ on its own and its task list is
checked here: every dependency is produced by an earlier task (so workgroups
taking tasks in list order can never deadlock), every task runs exactly
once, and executing the tasks in list order -- or in any order a set of
parallel workers could produce -- gives the Cholesky factor and its inverse.
"""
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sub_bit_weight_lb_amd", "csrc")

MAIN = r'''
#include <cstdio>
#include <cstdlib>
#include "chol_schedule.h"
int main(int argc, char** argv) {
  int R = std::atoi(argv[1]);
  auto t = nq::build_chol_schedule(R);
  for (auto& x : t) {
    std::printf("%d %d %d %d", x.type, x.i, x.j, x.k);
    for (auto& d : nq::chol_task_deps(x)) std::printf(" %d %d %d %d", d.kind, d.i, d.j, d.version);
    std::printf("\n");
  }
}
'''


@pytest.fixture(scope="module")
def sched_exe(tmp_path_factory):
    d = tmp_path_factory.mktemp("sched")
    src = d / "main.cpp"
    src.write_text(MAIN)
    exe = d / "sched"
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src),
                           os.path.join(CSRC, "chol_schedule.cpp"), "-o", str(exe)])
    return str(exe)


def schedule(exe, R):
    out = subprocess.check_output([exe, str(R)], text=True).strip().splitlines()
    tasks = []
    for line in out:
        v = list(map(int, line.split()))
        deps = [tuple(v[p:p + 4]) for p in range(4, len(v), 4)]
        tasks.append((tuple(v[:4]), deps))
    return tasks


def produces(task):
    t, i, j, k = task
    if t == 0:
        out = [(1, k, k, 1), (3, k, k, 1)]
        if k >= 1:
            out += [(1, k, k - 1, 1), (0, k, k, k)]
        return out
    if t == 1:
        return [(1, i, k, 1)]
    if t == 2:
        return [(3, k, j, 1)]
    if t == 3:
        return [(0, i, j, k + 1)]
    return [(2, i, j, k - j + 1)]


@pytest.mark.parametrize("R", [1, 2, 3, 5, 8, 17])
def test_dependencies_precede_and_tasks_are_complete(sched_exe, R):
    tasks = schedule(sched_exe, R)
    expect = R + sum(max(0, R - k - 2) for k in range(R)) + sum(k for k in range(R))
    expect += sum((R - k - 1) * (R - k) // 2 - (1 if k + 1 < R else 0) for k in range(R))
    expect += sum((R - k - 1) * (k + 1) for k in range(R))
    assert len(tasks) == expect
    assert len(set(t for t, _ in tasks)) == len(tasks)
    have = set()
    for t, deps in tasks:
        for d in deps:
            assert d in have, (t, d)
        have.update(produces(t))


def run_tasks(G, order, nb):
    """Execute tasks (fp64) in the given order on 64-blocked copies."""
    R = G.shape[0] // nb
    A = G.copy()
    M = np.zeros_like(G)
    blk = lambda X, a, b: X[a * nb:(a + 1) * nb, b * nb:(b + 1) * nb]
    for (t, i, j, k) in order:
        if t == 0:
            if k >= 1:
                L = blk(A, k, k - 1) @ blk(M, k - 1, k - 1).T
                blk(A, k, k - 1)[:] = L
                blk(A, k, k)[:] -= L @ L.T
            Lkk = np.linalg.cholesky(blk(A, k, k))
            blk(A, k, k)[:] = Lkk
            blk(M, k, k)[:] = np.linalg.inv(Lkk)
        elif t == 1:
            blk(A, i, k)[:] = blk(A, i, k) @ blk(M, k, k).T
        elif t == 2:
            blk(M, k, j)[:] = -blk(M, k, k) @ blk(M, k, j)
        elif t == 3:
            blk(A, i, j)[:] -= blk(A, i, k) @ blk(A, j, k).T
        else:
            blk(M, i, j)[:] += blk(A, i, k) @ blk(M, k, j)
    return np.tril(A), np.tril(M)


@pytest.mark.parametrize("R", [1, 2, 4, 7])
def test_list_order_computes_cholesky_and_inverse(sched_exe, R):
    nb = 4
    rng = np.random.default_rng(R)
    V = rng.standard_normal((3 * R * nb, R * nb))
    G = V.T @ V + np.eye(R * nb)
    tasks = [t for t, _ in schedule(sched_exe, R)]
    L, M = run_tasks(G, tasks, nb)
    np.testing.assert_allclose(L, np.linalg.cholesky(G), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(M @ L, np.eye(R * nb), atol=1e-10)


@pytest.mark.parametrize("workers,seed", [(3, 0), (16, 1), (64, 2)])
def test_parallel_workers_never_deadlock(sched_exe, workers, seed):
    """Workers take tickets in list order and run a task once its inputs exist;
    random task durations. Every run must finish and give the same factor."""
    R, nb = 6, 4
    tasks = schedule(sched_exe, R)
    rng = np.random.default_rng(seed)
    have = set()
    next_ticket = 0
    busy = {}          # worker -> (finish time, task index)
    waiting = {}       # worker -> task index
    now = 0.0
    done_order = []
    while len(done_order) < len(tasks):
        for w in range(workers):
            if w not in busy and w not in waiting and next_ticket < len(tasks):
                waiting[w] = next_ticket
                next_ticket += 1
        for w, n in list(waiting.items()):
            if all(d in have for d in tasks[n][1]):
                busy[w] = (now + rng.uniform(0.5, 2.0), n)
                del waiting[w]
        assert busy, "deadlock: every worker waits"
        w, (tf, n) = min(busy.items(), key=lambda kv: kv[1][0])
        now = tf
        del busy[w]
        have.update(produces(tasks[n][0]))
        done_order.append(tasks[n][0])
    V = np.random.default_rng(9).standard_normal((40, R * nb))
    G = V.T @ V + np.eye(R * nb)
    L, M = run_tasks(G, done_order, nb)
    np.testing.assert_allclose(L, np.linalg.cholesky(G), rtol=1e-10, atol=1e-12)


MAIN_DEV = r'''
#include <cstdio>
#include <cstdlib>
#include "chol_schedule.h"
int main(int argc, char** argv) {
  int R = std::atoi(argv[1]);
  for (auto& x : nq::build_chol_dev_tasks(R)) {
    std::printf("%d %d %d %d", x.type, x.i, x.j, x.k);
    for (int q = 0; q < 3; ++q) std::printf(" %d %d", x.dep[q], x.dver[q]);
    for (int q = 0; q < 3; ++q) std::printf(" %d %d", x.out[q], x.over[q]);
    std::printf("\n");
  }
}
'''


@pytest.mark.parametrize("R", [1, 2, 5, 12])
def test_device_records_waits_are_set_earlier(tmp_path, R):
    """Flag indices and versions in the device records: every wait targets a
    (flag, version) some earlier task sets, versions of one flag are set in
    increasing order, and no flag version is set twice."""
    src = tmp_path / "m.cpp"
    src.write_text(MAIN_DEV)
    exe = tmp_path / "m"
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-I", CSRC, str(src),
                           os.path.join(CSRC, "chol_schedule.cpp"), "-o", str(exe)])
    rows = [list(map(int, l.split()))
            for l in subprocess.check_output([str(exe), str(R)], text=True).splitlines()]
    setv = {}
    seen = set()
    for v in rows:
        deps = [(v[4 + 2 * q], v[5 + 2 * q]) for q in range(3)]
        outs = [(v[10 + 2 * q], v[11 + 2 * q]) for q in range(3)]
        for f, ver in deps:
            if f >= 0:
                assert 0 <= f < 4 * R * R and ver >= 1
                assert setv.get(f, 0) >= ver, (v, f, ver)
        for f, ver in outs:
            if f >= 0:
                assert (f, ver) not in seen
                seen.add((f, ver))
                assert ver == setv.get(f, 0) + 1 or (ver == 1 and f not in setv)
                setv[f] = max(setv.get(f, 0), ver)
