"""Comparison helpers shared by the tests (no GDN arithmetic here)."""
import numpy as np

REL = 1e-5      # per-element relative tolerance on o and S
FLOOR = 1e-6    # absolute floor for elements produced by cancellation


def tol_violations(x, r, rel=REL, floor=FLOOR):
    """Count of elements with |x - r| > max(rel*|r|, floor); floor may be an
    array broadcast against r."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    bad = np.abs(x - r) > np.maximum(rel * np.abs(r), floor)
    bad |= np.isnan(x) != np.isnan(r)
    return int(np.count_nonzero(bad))


def assert_close(x, r, what="", rel=REL, floor=FLOOR):
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    assert x.shape == r.shape, (what, x.shape, r.shape)
    n = tol_violations(x, r, rel, floor)
    if n:
        err = np.abs(x - r)
        i = int(np.argmax(err - np.broadcast_to(np.maximum(rel * np.abs(r), floor), err.shape)))
        raise AssertionError(
            f"{what}: {n}/{x.size} elements out of tolerance; worst at flat index "
            f"{i}: got {x.ravel()[i]!r} want {r.ravel()[i]!r}")


def max_rel_pages(x, r):
    """max |x - r| / max |r|: the per-token error metric printed with the
    f32 layer check of "Kestrel_VLLM #24", section 6."""
    x = np.asarray(x, np.float64)
    r = np.asarray(r, np.float64)
    den = np.max(np.abs(r))
    return float(np.max(np.abs(x - r)) / den) if den > 0 else float(np.max(np.abs(x - r)))


def bits_equal(a, b):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    return a.shape == b.shape and a.tobytes() == b.tobytes()


def host_threads():
    """Host threads for oracle work: the process's CPU share, at most 16."""
    import os
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return max(1, min(16, n or 1))


def over_unit_chunks(fn, n_units, chunk):
    """Run fn(lo, hi) for consecutive unit ranges of `chunk` units on a pool
    of host threads (the oracle releases the GIL), in order of the ranges;
    returns the list of results.  Only `host_threads()` ranges are in flight
    at once, so host memory stays bounded by what fn holds for one range."""
    from concurrent.futures import ThreadPoolExecutor
    ranges = [(lo, min(lo + chunk, n_units)) for lo in range(0, n_units, chunk)]
    with ThreadPoolExecutor(host_threads()) as ex:
        return list(ex.map(lambda r: fn(*r), ranges))


class Tally:
    """Elements out of tolerance and the pages' max|err| / max|ref| of one
    output over many chunks (combined from per-chunk maxima)."""

    def __init__(self):
        self.bad = 0
        self.n = 0
        self.max_err = 0.0
        self.max_ref = 0.0

    def add(self, x, r, rel=REL, floor=FLOOR):
        x = np.asarray(x, np.float64)
        r = np.asarray(r, np.float64)
        assert x.shape == r.shape, (x.shape, r.shape)
        self.bad += tol_violations(x, r, rel, floor)
        self.n += x.size
        if x.size:
            self.max_err = max(self.max_err, float(np.max(np.abs(x - r))))
            self.max_ref = max(self.max_ref, float(np.max(np.abs(r))))

    def merge(self, other):
        self.bad += other.bad
        self.n += other.n
        self.max_err = max(self.max_err, other.max_err)
        self.max_ref = max(self.max_ref, other.max_ref)

    @property
    def max_rel(self):
        return self.max_err / self.max_ref if self.max_ref > 0 else self.max_err

    def __repr__(self):
        return f"{self.bad}/{self.n} out of tolerance, max|err|/max|ref| = {self.max_rel:.3e}"
