"""A pool of CPU worker processes that run the oracle over chunks of a
full-size workload and compare every chunk with the HIP library's output.

The workers are started with the "spawn" method (fresh interpreters, never
a fork of a process that holds the GPU), use one BLAS thread each, and
import only numpy and the oracle (the task functions are in
fullsize_tasks.py).  Arrays travel through .npy files in a temporary
directory that the workers memory-map, so no large array is pickled; each
task returns a small dict of mismatch counts."""
import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np

_THREAD_VARS = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")


def worker_count(cap=16):
    """Workers for this host: the CPUs this process may run on, at most cap."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(cap, n))


class OraclePool:
    def __init__(self, n=None):
        self.n = n or worker_count()
        self.dir = tempfile.mkdtemp(prefix="fp4_oracle_")
        saved = {k: os.environ.get(k) for k in _THREAD_VARS}
        for k in _THREAD_VARS:
            os.environ[k] = "1"
        try:
            self.pool = mp.get_context("spawn").Pool(self.n)
        finally:
            for k, v in saved.items():
                if v is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = v

    def path(self, name):
        return os.path.join(self.dir, name + ".npy")

    def put(self, name, arr):
        """Writes arr to name.npy and returns its path."""
        p = self.path(name)
        np.save(p, np.ascontiguousarray(arr))
        return p

    def new(self, name, shape, dtype):
        """An uninitialised .npy array that workers fill in place."""
        p = self.path(name)
        np.lib.format.open_memmap(p, mode="w+", dtype=dtype, shape=tuple(shape)).flush()
        return p

    def get(self, path):
        return np.load(path, mmap_mode="r")

    def drop(self, *paths):
        for p in paths:
            if p and os.path.exists(p):
                os.remove(p)

    def map(self, fn, tasks):
        return self.pool.map(fn, tasks, chunksize=1)

    def close(self):
        self.pool.terminate()
        self.pool.join()
        shutil.rmtree(self.dir, ignore_errors=True)

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def spans(n, parts):
    """[a, b) ranges covering 0..n in about `parts` nearly equal pieces."""
    parts = max(1, min(parts, n))
    edges = np.linspace(0, n, parts + 1).round().astype(np.int64)
    return [(int(a), int(b)) for a, b in zip(edges[:-1], edges[1:]) if b > a]


def total(results, key):
    return sum(r[key] for r in results)


def first_bad(results, key):
    """The first reported mismatch location for key, or None."""
    for r in results:
        if r[key] and r.get(key + "_at") is not None:
            return r[key + "_at"]
    return None
