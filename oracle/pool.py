"""Run independent oracle tasks on a thread pool (CPU oracle; test infrastructure only).

Holds no arithmetic of the method.  The oracle's expert GEMMs are independent
per (expert, block of rows): each task writes rows no other task writes, so the
results do not depend on the number of workers or on the order in which tasks
finish.  With more than one worker, numpy's BLAS is held to one thread per
task (threadpoolctl) so the pool does not oversubscribe the cores.
"""
import concurrent.futures
import contextlib
import os


def default_workers():
    """Host threads the oracle may use: the cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _blas_one_thread():
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover - threadpoolctl is optional
        return contextlib.nullcontext()
    return threadpool_limits(1)


def run(tasks, workers=1):
    """Call every zero-argument callable in `tasks`; with workers > 1 on a thread pool."""
    tasks = list(tasks)
    if workers <= 1 or len(tasks) <= 1:
        for t in tasks:
            t()
        return
    with _blas_one_thread(), concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for f in [ex.submit(t) for t in tasks]:
            f.result()


def row_chunks(n, chunk):
    """[(start, stop), ...] covering range(n) in pieces of at most `chunk` rows."""
    return [(s, min(n, s + chunk)) for s in range(0, n, chunk)]
