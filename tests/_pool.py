"""A pool of forked, single-threaded worker processes for the oracle side of
the full-size parity tests (a helper module, not collected by pytest).

Work items read the large arrays (inputs, device results copied to the
host) from ``shared``, which the parent fills before the pool forks: the
children inherit them and nothing large is pickled on the way in.  Each
worker limits its BLAS to one thread, so the pool uses the host's cores
once.  The children only run numpy; they never touch the GPU."""
import multiprocessing as mp
import os
import sys
import time
from concurrent.futures import ProcessPoolExecutor

shared = {}


def workers() -> int:
    """At most 14 workers (the parent plus 14 children stays within the
    box's limit on processes per GPU), and one core left to the parent."""
    return max(1, min(14, (os.cpu_count() or 2) - 1))


def _init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def run(fn, jobs, what=""):
    """[fn(*job) for job in jobs] in the pool, in job order, with a
    progress line about every 20 s (a long oracle run is never silent)."""
    ctx = mp.get_context("fork")
    out = []
    t0 = last = time.time()
    with ProcessPoolExecutor(max_workers=workers(), mp_context=ctx, initializer=_init) as ex:
        futs = [ex.submit(fn, *j) for j in jobs]
        for n, f in enumerate(futs):
            out.append(f.result())
            now = time.time()
            if now - last > 20 or n + 1 == len(futs):
                print(f"  {what}: {n + 1}/{len(futs)} jobs, {now - t0:.0f} s", flush=True)
                sys.stdout.flush()
                last = now
    return out
