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
