"""Host-side checks of the C ABI: the library loads, exports every entry point
that include/gdn.h declares, and its argument validation refuses bad calls
before anything is enqueued (so these tests need no GPU and never launch)."""
import ctypes as C
import json
import os
import re

import numpy as np
import pytest

import gated_deltanet_recurrent_amd as gdn
from tests.helpers import max_rel_pages

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "gdn.h")
GOLD = os.path.join(ROOT, "tests", "golden")

D128 = (48, 16, 128, 128)
FAKE = 0x7f0000000000        # 256-byte aligned stand-in address; never dereferenced
NULLS = C.c_void_p(None)


def fp(off=0):
    return C.c_void_p(FAKE + off)


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\**\s*(gdn_[a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_function():
    L = gdn.lib()
    names = declared_functions()
    assert set(names) == set(gdn.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n


def test_strerror_covers_codes():
    L = gdn.lib()
    for rc in (0, -1, -2, -3, -4):
        assert L.gdn_strerror(rc)
    assert b"unknown" in L.gdn_strerror(-99)


def step_call(S=None, q=None, k=None, v=None, g=None, beta=None, o=None, N=4, dims=D128):
    vh, kh, kd, vd = dims
    sb = N * vh * kd * vd * 4
    S = fp(0) if S is None else S
    q = fp(sb) if q is None else q
    k = fp(sb + (1 << 20)) if k is None else k
    v = fp(sb + (2 << 20)) if v is None else v
    g = fp(sb + (3 << 20)) if g is None else g
    beta = fp(sb + (4 << 20)) if beta is None else beta
    o = fp(sb + (5 << 20)) if o is None else o
    return gdn.lib().gdn_step(S, q, k, v, g, beta, o, N, vh, kh, kd, vd, NULLS)


def test_step_validation():
    L = gdn.lib()
    assert step_call(dims=(48, 16, 96, 96)) == gdn.GDN_EUNSUPPORTED
    assert step_call(dims=(48, 16, 128, 64)) == gdn.GDN_EUNSUPPORTED
    assert step_call(dims=(48, 15, 128, 128)) == gdn.GDN_EINVAL      # vh % kh
    assert step_call(N=-1) == gdn.GDN_EINVAL
    assert step_call(N=0) == gdn.GDN_OK                                 # no-op, nothing enqueued
    assert step_call(S=NULLS) == gdn.GDN_EINVAL
    assert step_call(q=fp(4 * 48 * 128 * 128 * 4 + 4)) == gdn.GDN_EINVAL  # misaligned
    assert step_call(g=NULLS) == gdn.GDN_EINVAL
    assert step_call(o=fp(1024)) == gdn.GDN_EINVAL                      # o inside S
    assert step_call(q=fp(4096)) == gdn.GDN_EINVAL                      # q inside S
    # launch too large: tiles x 256 lanes must fit 32 bits
    assert step_call(N=(1 << 32) // (256 * 48) + 1) == gdn.GDN_EUNSUPPORTED
    vh, kh, kd, vd = D128
    for M in (0, 65, -3):
        assert L.gdn_step_m(fp(0), fp(1 << 30), fp(2 << 30), fp(3 << 30), fp(4 << 30),
                            fp(5 << 30), fp(6 << 30), 4, M, vh, kh, kd, vd, NULLS) == gdn.GDN_EINVAL


def test_slab_bytes_and_init():
    L = gdn.lib()
    vh, kh, kd, vd = D128
    assert L.gdn_slab_bytes(0, vh, kh, kd, vd, 0) == gdn.GDN_EINVAL
    assert L.gdn_slab_bytes(4, vh, kh, kd, vd, 6) == gdn.GDN_EINVAL          # not a multiple of 4
    assert L.gdn_slab_bytes(4, vh, kh, 32, 32, 0) == gdn.GDN_EUNSUPPORTED
    nb = L.gdn_slab_bytes(3, vh, kh, kd, vd, 0)
    assert nb == 3 * vh * kd * vd * 4 + 256
    # a slab's units are replayed in one recurrence launch: the step's grid limit
    assert L.gdn_slab_bytes((1 << 32) // (1024 * vh) + 1, vh, kh, kd, vd, 0) == gdn.GDN_EUNSUPPORTED
    assert L.gdn_slab_bytes(1 << 40, vh, kh, kd, vd, 0) == gdn.GDN_EUNSUPPORTED
    assert L.gdn_slab_bytes(4, vh, kh, kd, vd, (1 << 24) + 4) == gdn.GDN_EUNSUPPORTED
    assert L.gdn_slab_bytes(4, vh, kh, kd, vd, 1 << 24) == 4 * vh * kd * vd * 4 + 4 * 4 * (1 << 24) + 256
    s = gdn.gdn_slab()
    assert L.gdn_slab_init(C.byref(s), fp(0), nb - 1, 3, vh, kh, kd, vd, 0) == gdn.GDN_ESTATE
    assert L.gdn_slab_init(C.byref(s), fp(16), nb, 3, vh, kh, kd, vd, 0) == gdn.GDN_EINVAL  # align
    assert L.gdn_slab_init(C.byref(s), fp(0), nb, 3, vh, kh, kd, vd, 0) == gdn.GDN_OK
    assert s.armed == 0 and s.n_units == 3


def test_slab_size_matches_pages_state_sizes():
    """The pages' own size figures for 48 layers of S and conv history."""
    gold = json.load(open(os.path.join(GOLD, "state_sizes_p24.json")))
    sh = gold["shape"]
    L = gdn.lib()
    n = sh["layers"]
    hist = (sh["ck"] - 1) * sh["conv_dim"]
    total = L.gdn_slab_bytes(n, sh["vh"], sh["kh"], sh["kd"], sh["vd"], hist)
    s_only = L.gdn_slab_bytes(n, sh["vh"], sh["kh"], sh["kd"], sh["vd"], 0)
    s_bytes = s_only - 256                       # minus the accepted[] area
    h_bytes = total - s_only
    assert round(s_bytes / 1e6, 1) == gold["state_S_MB"]
    assert round(h_bytes / 1e6, 1) == gold["conv_history_MB"]
    assert round((s_bytes + h_bytes) / 2**20, 1) == gold["state_plus_history_MiB"]


def test_rollback_refusals_need_no_device():
    L = gdn.lib()
    vh, kh, kd, vd = D128
    nb = L.gdn_slab_bytes(2, vh, kh, kd, vd, 3 * 10240)
    s = gdn.gdn_slab()
    assert L.gdn_slab_init(C.byref(s), fp(0), nb, 2, vh, kh, kd, vd, 3 * 10240) == 0
    acc = (C.c_int32 * 2)(0, 1)
    args = [fp(1 << 32), NULLS] + [fp((i + 2) << 32) for i in range(5)] + [NULLS]
    # never marked: one-shot state error
    assert L.gdn_rollback(C.byref(s), *args, 10240, 4, 4, acc, NULLS) == gdn.GDN_ESTATE
    # an uninitialised slab
    bad = gdn.gdn_slab()
    assert L.gdn_rollback(C.byref(bad), *args, 10240, 4, 4, acc, NULLS) == gdn.GDN_ESTATE
    assert L.gdn_mark(C.byref(bad), fp(1 << 32), NULLS, NULLS) == gdn.GDN_ESTATE
    # armed state only (history not marked): a history rollback is refused
    s.armed = 1
    args_h = list(args)
    args_h[1] = fp(9 << 32)
    assert L.gdn_rollback(C.byref(s), *args_h, 10240, 4, 4, acc, NULLS) == gdn.GDN_ESTATE
    # accepted out of range / M out of range
    acc_bad = (C.c_int32 * 2)(0, 5)
    assert L.gdn_rollback(C.byref(s), *args, 10240, 4, 4, acc_bad, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_rollback(C.byref(s), *args, 10240, 4, 0, acc, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_rollback(C.byref(s), *args, 10240, 4, 65, acc, NULLS) == gdn.GDN_EINVAL
    # S inside the slab
    args_s = list(args)
    args_s[0] = fp(4096)
    assert L.gdn_rollback(C.byref(s), *args_s, 10240, 4, 4, acc, NULLS) == gdn.GDN_EINVAL
    # the conv kernel width: only ck = 4 is built; ignored without a history
    s.armed = 3
    assert L.gdn_rollback(C.byref(s), *args_h, 10240, 3, 4, acc, NULLS) == gdn.GDN_EUNSUPPORTED
    assert L.gdn_rollback(C.byref(s), *args_h, 10240, 5, 4, acc, NULLS) == gdn.GDN_EUNSUPPORTED
    # the most units one launch takes, with a history replay that passes the grid limit
    n, cd = (1 << 32) // (1024 * vh), 1 << 22
    nb = L.gdn_slab_bytes(n, vh, kh, kd, vd, 3 * cd)
    assert nb > 0
    big = gdn.gdn_slab()
    assert L.gdn_slab_init(C.byref(big), fp(0), nb, n, vh, kh, kd, vd, 3 * cd) == 0
    big.armed = 3
    zeros = (C.c_int32 * n)()
    args_big = [fp(1 << 44), fp(1 << 45)] + [NULLS] * 6
    assert L.gdn_rollback(C.byref(big), *args_big, cd, 4, 4, zeros, NULLS) == gdn.GDN_EUNSUPPORTED
    # history size disagreeing with the slab's (conv_dim * (ck - 1))
    assert L.gdn_rollback(C.byref(s), *args_h, 10236, 4, 4, acc, NULLS) == gdn.GDN_EINVAL
    assert s.armed == 3        # refusals leave the slab as it was


def test_mark_step_m_refusals_need_no_device():
    L = gdn.lib()
    vh, kh, kd, vd = D128
    nb = L.gdn_slab_bytes(2, vh, kh, kd, vd, 0)
    s = gdn.gdn_slab()
    assert L.gdn_slab_init(C.byref(s), fp(0), nb, 2, vh, kh, kd, vd, 0) == 0
    ptrs = [fp((i + 2) << 32) for i in range(7)]   # S, q, k, v, g, beta, o
    args = [ptrs[0], NULLS] + ptrs[1:]
    assert L.gdn_mark_step_m(C.byref(gdn.gdn_slab()), *args, 2, 4, vh, kh, kd, vd, NULLS) == gdn.GDN_ESTATE
    assert L.gdn_mark_step_m(C.byref(s), *args, 3, 4, vh, kh, kd, vd, NULLS) == gdn.GDN_ESTATE
    assert L.gdn_mark_step_m(C.byref(s), *args, 2, 4, vh, kh, 64, 64, NULLS) == gdn.GDN_ESTATE
    assert L.gdn_mark_step_m(C.byref(s), *args, 2, 0, vh, kh, kd, vd, NULLS) == gdn.GDN_EINVAL
    args_h = [ptrs[0], fp(9 << 32)] + ptrs[1:]     # history given, slab has none
    assert L.gdn_mark_step_m(C.byref(s), *args_h, 2, 4, vh, kh, kd, vd, NULLS) == gdn.GDN_ESTATE
    assert s.armed == 0


def test_verify_commit_refusals_need_no_device():
    L = gdn.lib()
    vh, kh, kd, vd = D128
    ptrs = [fp((i + 2) << 32) for i in range(9)]
    S, q, k, v, g, beta, o, xc, hist = ptrs
    assert L.gdn_verify_m(S, q, k, v, g, beta, o, 4, 0, vh, kh, kd, vd, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_verify_m(S, q, k, v, g, beta, fp((2 << 32) + 4096), 4, 2, vh, kh, kd, vd,
                          NULLS) == gdn.GDN_EINVAL                   # o inside S
    acc = fp(20 << 32)
    assert L.gdn_commit(S, NULLS, q, k, v, g, beta, NULLS, 0, 4, 4, 2, vh, kh, kd, vd, NULLS, NULLS,
                        NULLS) == gdn.GDN_EINVAL                       # no accepted array
    assert L.gdn_commit(S, NULLS, q, k, v, g, beta, NULLS, 0, 4, 4, 2, vh, kh, kd, vd,
                        fp((20 << 32) + 2), NULLS, NULLS) == gdn.GDN_EINVAL   # misaligned
    assert L.gdn_commit(S, hist, q, k, v, g, beta, NULLS, 10240, 4, 4, 2, vh, kh, kd, vd, acc, NULLS,
                        NULLS) == gdn.GDN_EINVAL                       # history without raws
    assert L.gdn_commit(S, NULLS, q, k, v, g, beta, NULLS, 0, 4, 4, 65, vh, kh, kd, vd, acc, NULLS,
                        NULLS) == gdn.GDN_EINVAL
    assert L.gdn_commit(S, NULLS, q, k, v, g, beta, NULLS, 0, 4, 0, 2, vh, kh, kd, vd, acc, NULLS,
                        NULLS) == gdn.GDN_OK                           # nothing to do
    assert L.gdn_commit(S, hist, q, k, v, g, beta, xc, 10240, 3, 4, 2, vh, kh, kd, vd, acc, NULLS,
                        NULLS) == gdn.GDN_EUNSUPPORTED                 # conv width 3 not built
    # the written history inside an input row array; status inside accepted or the history
    assert L.gdn_commit(S, fp((3 << 32) + 1024), q, k, v, g, beta, xc, 10240, 4, 4, 2, vh, kh,
                        kd, vd, acc, NULLS, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_commit(S, fp((6 << 32) + 16), q, k, v, g, beta, xc, 10240, 4, 4, 2, vh, kh, kd,
                        vd, acc, NULLS, NULLS) == gdn.GDN_EINVAL      # inside g
    assert L.gdn_commit(S, NULLS, q, k, v, g, beta, NULLS, 0, 4, 4, 2, vh, kh, kd, vd, acc,
                        fp((20 << 32) + 4), NULLS) == gdn.GDN_EINVAL
    assert L.gdn_commit(S, hist, q, k, v, g, beta, xc, 10240, 4, 4, 2, vh, kh, kd, vd, acc,
                        fp((10 << 32) + 64), NULLS) == gdn.GDN_EINVAL
    # the fused commit + verify: M2 out of range; o inside S, inside a first-set
    # row array, or the history inside a second-set row array
    q2, k2, v2, g2, b2, o2 = (fp((40 + i) << 32) for i in range(6))
    cv = lambda S_, hist_, o_, M2_, q2_=q2: L.gdn_commit_verify_m(  # noqa: E731
        S_, hist_, q, k, v, g, beta, xc if hist_ else NULLS, 10240 if hist_ else 0, 4, 4, 2, acc,
        NULLS, q2_, k2, v2, g2, b2, o_, M2_, vh, kh, kd, vd, NULLS)
    assert cv(S, NULLS, o2, 0) == gdn.GDN_EINVAL
    assert cv(S, NULLS, o2, 65) == gdn.GDN_EINVAL
    assert cv(S, NULLS, fp((2 << 32) + 4096), 2) == gdn.GDN_EINVAL          # o inside S
    assert cv(S, NULLS, fp((5 << 32) + 512), 2) == gdn.GDN_EINVAL           # o inside v
    assert cv(S, hist, o2, 2, q2_=fp((10 << 32) + 256)) == gdn.GDN_EINVAL   # q2 inside the history
    assert cv(S, NULLS, o2, 2, q2_=NULLS) == gdn.GDN_EINVAL
    assert L.gdn_commit_verify_m(S, NULLS, q, k, v, g, beta, NULLS, 0, 4, 0, 2, acc, NULLS, q2, k2,
                                 v2, g2, b2, o2, 2, vh, kh, kd, vd, NULLS) == gdn.GDN_OK
    # the history replay's workgroups count towards the grid limit: 64 units of
    # 2^28 channels need 2^32 replay lanes
    assert L.gdn_commit(S, hist, q, k, v, g, beta, xc, 1 << 28, 4, 64, 2, vh, kh, kd, vd, acc,
                        NULLS, NULLS) == gdn.GDN_EUNSUPPORTED
    z, w = fp(30 << 32), fp(31 << 32)
    eps = C.c_float(1e-6)
    assert L.gdn_verify_m_gated(S, q, k, v, g, beta, z, w, eps, o, 4, 0, vh, kh, kd, vd,
                                NULLS) == gdn.GDN_EINVAL                # M = 0
    assert L.gdn_verify_m_gated(S, q, k, v, g, beta, z, w, C.c_float(float("nan")), o, 4, 2,
                                vh, kh, kd, vd, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_verify_m_gated(S, q, k, v, g, beta, z, w, eps, fp((30 << 32) + 1024), 4, 2,
                                vh, kh, kd, vd, NULLS) == gdn.GDN_EINVAL  # out overlaps z
    assert L.gdn_verify_m_gated(S, q, k, v, g, beta, NULLS, w, eps, o, 4, 2, vh, kh, kd, vd,
                                NULLS) == gdn.GDN_EINVAL                # no gate
    assert L.gdn_verify_m_gated(S, q, k, v, g, beta, z, w, eps, o, 0, 2, vh, kh, kd, vd,
                                NULLS) == gdn.GDN_OK                    # nothing to do


def test_frontend_validation():
    L = gdn.lib()
    vh, kh, kd, vd = D128
    ptrs = [fp(i << 32) for i in range(13)]
    cd = 2 * kh * kd + vh * vd
    assert L.gdn_frontend(*ptrs, 4, 5120, cd + 4, 4, vh, kh, kd, vd, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_frontend(*ptrs, 4, 5120, cd, 3, vh, kh, kd, vd, NULLS) == gdn.GDN_EUNSUPPORTED
    assert L.gdn_frontend(*ptrs, 4, 5122, cd, 4, vh, kh, kd, vd, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_frontend(*ptrs, 0, 5120, cd, 4, vh, kh, kd, vd, NULLS) == gdn.GDN_OK
    p2 = list(ptrs)
    p2[9] = p2[8]                                   # k aliases q
    assert L.gdn_frontend(*p2, 4, 5120, cd, 4, vh, kh, kd, vd, NULLS) == gdn.GDN_EINVAL
    # an output or the history inside a weight input
    # (x, Wa, Wb, A_log, dt_bias, xc_raw, hist, conv_w, q, k, v, g, beta)
    for i, inside in ((8, (1 << 32) + 256), (10, (2 << 32) + 4096), (11, 3 << 32),
                      (12, 4 << 32), (6, (7 << 32) + 64), (6, 16)):
        p2 = list(ptrs)
        p2[i] = fp(inside)
        assert L.gdn_frontend(*p2, 4, 5120, cd, 4, vh, kh, kd, vd, NULLS) == gdn.GDN_EINVAL, i


def test_stream_read_validation():
    L = gdn.lib()
    assert L.gdn_stream_read_words(0) < 0
    assert L.gdn_stream_read_words(1) == 1
    assert L.gdn_stream_read_words(32768) == 1
    assert L.gdn_stream_read_words(32769) == 2
    assert L.gdn_stream_read(fp(0), 100, fp(64), NULLS) == gdn.GDN_EINVAL    # words inside src
    assert L.gdn_stream_read(fp(0), 100, fp((1 << 20) + 2),
                             NULLS) == gdn.GDN_EINVAL                        # misaligned words
    assert L.gdn_stream_read(fp(8), 100, fp(1 << 20), NULLS) == gdn.GDN_EINVAL  # src not 16-aligned
    assert L.gdn_stream_read(fp(0), -1, fp(1 << 20), NULLS) == gdn.GDN_EINVAL
    assert L.gdn_stream_read(fp(0), 0, fp(1 << 20), NULLS) == gdn.GDN_OK


def test_stream_copy_validation():
    L = gdn.lib()
    assert L.gdn_stream_copy(fp(0), fp(64), 100, NULLS) == gdn.GDN_EINVAL   # overlap
    assert L.gdn_stream_copy(fp(0), fp(1 << 20), -1, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_stream_copy(fp(0), fp(1 << 20), 0, NULLS) == gdn.GDN_OK


def test_proj_validation():
    """gdn_proj refuses bad shapes, pointers and overlaps before any launch."""
    L = gdn.lib()
    x, W0, y0, W1, y1 = (fp(i << 36) for i in range(5))
    ok = (x, 4, 5120, W0, 10240, y0, W1, 6144, y1, NULLS)
    args = list(ok)
    args[2] = 5120 + 64                                  # C not a multiple of 128
    assert L.gdn_proj(*args) == gdn.GDN_EUNSUPPORTED
    args = list(ok)
    args[4] = 10248                                      # R0 not a multiple of 16
    assert L.gdn_proj(*args) == gdn.GDN_EUNSUPPORTED
    args = list(ok)
    args[7] = 6152
    assert L.gdn_proj(*args) == gdn.GDN_EUNSUPPORTED
    for i, bad in ((1, -1), (2, 0), (4, 0), (7, 0)):
        args = list(ok)
        args[i] = bad
        assert L.gdn_proj(*args) == gdn.GDN_EINVAL, (i, bad)
    assert L.gdn_proj(x, 4, 5120, W0, 10240, y0, NULLS, 16, NULLS, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj(x, 4, 5120, W0, 10240, y0, NULLS, 0, y1, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj(x, 4, 5120, NULLS, 10240, y0, NULLS, 0, NULLS, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj(fp(4), 4, 5120, W0, 10240, y0, NULLS, 0, NULLS, NULLS) == gdn.GDN_EINVAL
    # outputs overlapping an input or each other
    assert L.gdn_proj(x, 4, 5120, W0, 10240, fp(64), NULLS, 0, NULLS, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj(x, 4, 5120, W0, 10240, y0, W1, 6144, fp((2 << 36) + 256),
                      NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj(x, 4, 5120, W0, 10240, y0, W1, 6144, fp((3 << 36) + 1024),
                      NULLS) == gdn.GDN_EINVAL
    # sizes beyond the 32-bit weight addressing or the grid are refused
    assert L.gdn_proj(x, 4, (1 << 22) + 128, W0, 16, y0, NULLS, 0, NULLS,
                      NULLS) == gdn.GDN_EUNSUPPORTED
    assert L.gdn_proj(x, (1 << 31) + 1, 5120, W0, 16, y0, NULLS, 0, NULLS,
                      NULLS) == gdn.GDN_EUNSUPPORTED
    # no rows: nothing to do, nothing launched
    assert L.gdn_proj(x, 0, 5120, W0, 10240, y0, W1, 6144, y1, NULLS) == gdn.GDN_OK


def test_proj_pack_validation():
    L = gdn.lib()
    W, Wp = fp(0), fp(1 << 36)
    assert L.gdn_proj_pack(W, Wp, 10240, 5120 + 64, NULLS) == gdn.GDN_EUNSUPPORTED
    assert L.gdn_proj_pack(W, Wp, 10248, 5120, NULLS) == gdn.GDN_EUNSUPPORTED
    assert L.gdn_proj_pack(W, Wp, 0, 5120, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj_pack(W, Wp, 16, -128, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj_pack(W, fp(4096), 16, 128, NULLS) == gdn.GDN_EINVAL     # overlap
    assert L.gdn_proj_pack(fp(8), Wp, 16, 128, NULLS) == gdn.GDN_EINVAL       # misaligned
    assert L.gdn_proj_pack(NULLS, Wp, 16, 128, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj_pack(W, Wp, 16, (1 << 22) + 128, NULLS) == gdn.GDN_EUNSUPPORTED
    assert L.gdn_proj_pack(W, Wp, 1 << 30, 1 << 12, NULLS) == gdn.GDN_EUNSUPPORTED


def test_max_rel_metric_matches_pages_row():
    gold = json.load(open(os.path.join(GOLD, "max_rel_p24.json")))
    r = np.array([gold["max_abs_ref"], -3.0, 1.0])
    x = r + np.array([gold["max_abs_err"], 1e-7, -5e-7])
    assert abs(max_rel_pages(x, r) - gold["max_rel"]) / gold["max_rel"] < 2e-3


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(gdn, "_lib", None)
    monkeypatch.setattr(gdn, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(ImportError):
        gdn.lib()


def test_proj_q4_bytes():
    """Packed 4-bit size: C/2 bytes of values and C/32 binary16 scales per row."""
    L = gdn.lib()
    assert L.gdn_proj_q4_bytes(10240, 5120) == 10240 * (5120 // 2 + 5120 // 32 * 2)
    assert L.gdn_proj_q4_bytes(64, 1024) == 64 * 576
    for R, Cc in ((0, 1024), (64, 0), (16, 1024), (96, 1024), (64, 512), (64, 1536), (-64, 1024)):
        assert L.gdn_proj_q4_bytes(R, Cc) == -1, (R, Cc)


def test_smoke_shapes_pass_host_validation():
    """The 4-bit projection smoke() runs has a shape the library accepts (the
    size query validates it on the host, no GPU needed)."""
    import __graft_entry__ as entry
    rows, R, Cc = entry.SMOKE_Q4
    assert 1 <= rows <= 16
    assert gdn.lib().gdn_proj_q4_bytes(R, Cc) == R * (Cc // 2 + Cc // 32 * 2)


def test_proj_q4_pack_validation():
    L = gdn.lib()
    q, sc, Wq = fp(0), fp(1 << 36), fp(2 << 36)
    assert L.gdn_proj_q4_pack(q, sc, Wq, 10240, 5120 + 128, NULLS) == gdn.GDN_EUNSUPPORTED
    assert L.gdn_proj_q4_pack(q, sc, Wq, 10240 + 16, 5120, NULLS) == gdn.GDN_EUNSUPPORTED
    assert L.gdn_proj_q4_pack(q, sc, Wq, 64, (1 << 22) + 1024, NULLS) == gdn.GDN_EUNSUPPORTED
    assert L.gdn_proj_q4_pack(q, sc, Wq, 0, 5120, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj_q4_pack(q, sc, Wq, 64, -1024, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj_q4_pack(NULLS, sc, Wq, 64, 1024, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj_q4_pack(q, fp(8), Wq, 64, 1024, NULLS) == gdn.GDN_EINVAL   # misaligned
    # the packed output (64 * 576 bytes) overlapping the values or the scales
    assert L.gdn_proj_q4_pack(q, sc, fp(8192), 64, 1024, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj_q4_pack(q, sc, fp((1 << 36) + 256), 64, 1024, NULLS) == gdn.GDN_EINVAL


def test_proj_q4_validation():
    """gdn_proj_q4 refuses bad shapes, more than 16 rows, bad pointers and
    overlaps before any launch."""
    L = gdn.lib()
    x, W0, y0, W1, y1 = (fp(i << 36) for i in range(5))
    ok = (x, 4, 5120, W0, 10240, y0, W1, 6144, y1, NULLS)
    for i, bad in ((2, 5120 + 128), (2, 5120 + 512), (4, 10248), (4, 10240 + 16), (7, 6144 + 32),
                   (1, 17)):
        args = list(ok)
        args[i] = bad
        assert L.gdn_proj_q4(*args) == gdn.GDN_EUNSUPPORTED, (i, bad)
    for i, bad in ((1, -1), (2, 0), (4, 0), (7, 0)):
        args = list(ok)
        args[i] = bad
        assert L.gdn_proj_q4(*args) == gdn.GDN_EINVAL, (i, bad)
    assert L.gdn_proj_q4(x, 4, 5120, W0, 10240, y0, NULLS, 16, NULLS, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj_q4(x, 4, 5120, W0, 10240, y0, NULLS, 0, y1, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj_q4(x, 4, 5120, NULLS, 10240, y0, NULLS, 0, NULLS, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj_q4(fp(4), 4, 5120, W0, 10240, y0, NULLS, 0, NULLS,
                         NULLS) == gdn.GDN_EINVAL
    # outputs overlapping the packed weights (10240 x 5120 x 9/16 bytes) or each other
    assert L.gdn_proj_q4(x, 4, 5120, W0, 10240, fp((1 << 36) + 29491200 - 16), NULLS, 0,
                         NULLS, NULLS) == gdn.GDN_EINVAL
    assert L.gdn_proj_q4(x, 4, 5120, W0, 10240, y0, W1, 6144, fp((2 << 36) + 256),
                         NULLS) == gdn.GDN_EINVAL
    # the end of the weights just before y0 is no overlap; no rows is a no-op
    assert L.gdn_proj_q4(x, 0, 5120, W0, 10240, y0, W1, 6144, y1, NULLS) == gdn.GDN_OK
