"""The fp64 oracle over a whole full-size output, in worker processes.

Test infrastructure (not collected: no test_ prefix).  The oracle itself is
unchanged: ``oracle.decode_attention`` runs on sub-batches of queries, each in
a freshly spawned worker process that never touches the GPU.

Why workers: the plain oracle gathers each (query, kv head) pair's whole
context (prefix ++ distinct) page by page, a single-threaded memory copy of
up to 11 MB per pair at the LongChat-like shape.  Spread over the host's
cores it takes seconds instead of minutes.

Data path: the parent writes the raw bits of q and of the two pools once
into a temporary directory (bf16 as uint16, fp32 as float32).  Each worker
memory-maps them, copies out the pages its queries name
(``workloads.subset_for_queries``), widens them exactly to float64 (bf16:
the bits shifted into the high half of a float32), and calls the oracle.
"""

from __future__ import annotations

import multiprocessing as mp
import os
import shutil
import tempfile
import time

import numpy as np

_W = {}


def host_workers():
    """Worker count: the cores this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _widen(a, bf16):
    """Exact float64 values of raw bf16 (uint16) or fp32 elements."""
    if bf16:
        a = (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    return np.asarray(a, dtype=np.float64)


def _init(dirname, bf16, shapes, batch, scale):
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except Exception:  # pragma: no cover - BLAS threads only affect speed
        pass
    dt = np.uint16 if bf16 else np.float32
    _W["q"] = np.memmap(os.path.join(dirname, "q.bin"), dtype=dt, mode="r", shape=shapes[0])
    _W["k"] = np.memmap(os.path.join(dirname, "k.bin"), dtype=dt, mode="r", shape=shapes[1])
    _W["v"] = np.memmap(os.path.join(dirname, "v.bin"), dtype=dt, mode="r", shape=shapes[2])
    _W["bf16"] = bf16
    _W["batch"] = batch
    _W["scale"] = scale


def _job(queries):
    import oracle
    from workloads import subset_for_queries

    bf16 = _W["bf16"]
    sub, page_ids = subset_for_queries(_W["batch"], queries)
    ks = _widen(_W["k"][page_ids], bf16)
    vs = _widen(_W["v"][page_ids], bf16)
    qs = _widen(_W["q"][np.asarray(queries, dtype=np.int64)], bf16)
    O, M, L = oracle.decode_attention(qs, ks, vs, sub, scale=_W["scale"])
    return queries, O, M, L


def _raw(t):
    """Host numpy view of a tensor's raw bits (uint16 for bf16, float32 for fp32)."""
    import torch

    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.contiguous().cpu().numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


def _scratch_dir(need_bytes):
    for base in ("/dev/shm", tempfile.gettempdir()):
        try:
            st = os.statvfs(base)
        except OSError:
            continue
        if st.f_bavail * st.f_frsize > need_bytes * 1.25 + (1 << 30) and os.access(base, os.W_OK):
            return tempfile.mkdtemp(prefix="psa_oracle_", dir=base)
    raise RuntimeError(f"no temporary space for {need_bytes / 2**30:.1f} GiB of oracle inputs")


def oracle_full(batch, q, k, v, chunk, scale=None, workers=None, log=print, what=""):
    """(O, M, L) of every query of ``batch`` in float64, via worker processes.

    ``q, k, v`` are device (or host) tensors in bf16 or fp32; ``chunk`` queries
    go to a worker at a time.  Prints progress at least every 20 s.
    """
    import torch

    bf16 = q.dtype == torch.bfloat16
    n = len(batch["query_group"])
    hq, d = int(q.shape[1]), int(q.shape[2])
    need = (q.numel() + k.numel() + v.numel()) * (2 if bf16 else 4)
    workers = workers or host_workers()
    tmp = _scratch_dir(need)
    O = np.zeros((n, hq, d))
    M = np.zeros((n, hq))
    L = np.zeros((n, hq))
    try:
        shapes = []
        for name, t in (("q", q), ("k", k), ("v", v)):
            a = _raw(t)
            shapes.append(a.shape)
            a.tofile(os.path.join(tmp, f"{name}.bin"))
            del a
        log(f"  oracle {what}: inputs written to {tmp}")
        plain = {key: (np.asarray(val) if not isinstance(val, (int, float)) else val) for key, val in batch.items()}
        chunks = [list(range(a, min(n, a + chunk))) for a in range(0, n, chunk)]
        ctx = mp.get_context("spawn")
        t0 = last = time.time()
        done = 0
        log(f"  oracle {what}: {n} queries in {len(chunks)} batches on {workers} worker processes")
        with ctx.Pool(workers, initializer=_init, initargs=(tmp, bf16, shapes, plain, scale)) as pool:
            for qs, o, m, l in pool.imap_unordered(_job, chunks):
                O[qs], M[qs], L[qs] = o, m, l
                done += len(qs)
                if time.time() - last > 20:
                    last = time.time()
                    log(f"  oracle {what}: {done}/{n} queries, {last - t0:.0f} s")
        log(f"  oracle {what}: {n} queries in {time.time() - t0:.1f} s")
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return O, M, L
