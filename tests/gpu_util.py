"""Helpers for the GPU parity tests: device placement and case announcements."""
import numpy as np
import torch


def dev() -> torch.device:
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def case(msg: str) -> None:
    """Name the case before its GPU work starts, so a lost run still says what it was doing."""
    print(f"[case] {msg}", flush=True)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def oracle_threads() -> int:
    """Host threads for whole-matrix oracle runs: the process's CPU share, at most 16."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_all_rows(fn, out_f: int):
    """Run a row-ranged oracle call fn(rows) -> (y, A) over every output row, with the rows split
    across host threads (the oracle is a C library; ctypes releases the GIL while it runs).
    Each thread writes a disjoint column range of the [m, out_f] results, so the merged arrays
    equal one call over all rows."""
    import concurrent.futures as cf
    nth = oracle_threads()
    step = (out_f + nth - 1) // nth
    ranges = [(r, min(out_f, r + step)) for r in range(0, out_f, step)]
    with cf.ThreadPoolExecutor(max_workers=nth) as ex:
        parts = list(ex.map(fn, ranges))
    y = parts[0][0].copy()
    A = parts[0][1].copy()
    for (r0, r1), (yp, Ap) in zip(ranges, parts):
        y[:, r0:r1] = yp[:, r0:r1]
        A[:, r0:r1] = Ap[:, r0:r1]
    return y, A
