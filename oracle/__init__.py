"""CPU oracle for the GDN recurrent decode step (ctypes over plain C).

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library and never imports it.

The arithmetic lives in ``gdn_oracle.c`` (fp32, separate rounding of every
operation, the stated loop order) and its double-precision brute-force twin
``ref64_gdn_step``.  This module only compiles that file with gcc and marshals
numpy arrays into it.

Sources: "Kestrel_VLLM #24: GDN linear attention on GPU" (Fig. 1 caption,
sections 3 and 4), "Kestrel_VLLM #27: register residency and fused launch"
(sections 3.1 and 4.2), "Kestrel_VLLM #34: batched M rows" (sections 3.6 and
3.7).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "gdn_oracle.c")
LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
# Plain scalar C: no FMA contraction, no re-association, no fast-math.
CFLAGS = ["-std=c99", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-Wall", "-Wextra"]


def build(verbose: bool = False, src: str = SRC, out: str = LIB_PATH) -> str:
    """Compile the oracle with gcc (default: into ``oracle/libgdn_oracle.so``)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, "-I", _HERE, "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class RefSlab(C.Structure):
    _fields_ = [("S_snap", C.c_void_p), ("hist_snap", C.c_void_p),
                ("n_units", C.c_int64), ("hist_floats", C.c_int64),
                ("vh", C.c_int), ("kh", C.c_int), ("kd", C.c_int),
                ("vd", C.c_int), ("armed", C.c_int)]


def _f32(a, name, writable=False):
    if not isinstance(a, np.ndarray) or a.dtype != np.float32 or not a.flags.c_contiguous:
        raise TypeError(f"{name}: need a C-contiguous float32 numpy array")
    if writable and not a.flags.writeable:
        raise TypeError(f"{name}: must be writable")
    return a.ctypes.data_as(C.c_void_p)


def _f64(a, name):
    if not isinstance(a, np.ndarray) or a.dtype != np.float64 or not a.flags.c_contiguous:
        raise TypeError(f"{name}: need a C-contiguous float64 numpy array")
    return a.ctypes.data_as(C.c_void_p)


def _opt(a, name):
    return None if a is None else _f32(a, name)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what}: oracle refused the arguments (rc={rc})")


class Oracle:
    """ctypes handle on one compiled copy of the oracle."""

    def __init__(self, path: str):
        lib = C.CDLL(path)
        P, I, L = C.c_void_p, C.c_int, C.c_int64
        lib.ref_gdn_step.argtypes = [P] * 7 + [L, I, I, I, I]
        lib.ref_gdn_step_m.argtypes = [P] * 7 + [L, I, I, I, I, I]
        lib.ref_gdn_mark.argtypes = [C.POINTER(RefSlab), P, P]
        lib.ref_gdn_rollback.argtypes = ([C.POINTER(RefSlab), P, P] + [P] * 5 +
                                         [P, I, I, I, P])
        lib.ref_conv_push.argtypes = [P, P, I, I]
        lib.ref_conv_push.restype = None
        lib.ref_gdn_frontend.argtypes = [P] * 13 + [I] * 8
        lib.ref_gdn_frontend_m.argtypes = [P] * 13 + [I] * 9
        lib.ref64_gdn_step.argtypes = [P] * 7 + [L, I, I, I, I]
        lib.ref_gdn_gated_norm.argtypes = [P, P, P, C.c_float, P, L, I]
        lib.ref_gdn_gated_norm.restype = C.c_int
        lib.ref_gdn_proj.argtypes = [P, P, P, L, I, I]
        lib.ref_gdn_proj.restype = C.c_int
        lib.ref_half_to_float.argtypes = [P, P, L]
        lib.ref_half_to_float.restype = None
        lib.ref_gdn_proj_q4.argtypes = [P, P, P, P, L, I, I]
        lib.ref_gdn_proj_q4.restype = C.c_int
        for f in ("ref_gdn_step", "ref_gdn_step_m", "ref_gdn_mark", "ref_gdn_rollback",
                  "ref_gdn_frontend", "ref_gdn_frontend_m", "ref64_gdn_step"):
            getattr(lib, f).restype = C.c_int
        self.lib = lib
        self.path = path

    def gdn_step(self, S, q, k, v, g, beta, o, dims, n_units=None):
        """One step for every unit; S [N][vh][kd][vd] and o [N][vh][vd] in place."""
        vh, kh, kd, vd = dims
        n = S.size // (vh * kd * vd) if n_units is None else n_units
        rc = self.lib.ref_gdn_step(_f32(S, "S", True), _f32(q, "q"), _f32(k, "k"),
                                   _f32(v, "v"), _f32(g, "g"), _f32(beta, "beta"),
                                   _f32(o, "o", True), n, vh, kh, kd, vd)
        _check(rc, "ref_gdn_step")

    def gdn_step_m(self, S, q, k, v, g, beta, o, M, dims):
        """M sequential steps; inputs [M][N][...], o [M][N][vh][vd]."""
        vh, kh, kd, vd = dims
        n = S.size // (vh * kd * vd)
        rc = self.lib.ref_gdn_step_m(_f32(S, "S", True), _f32(q, "q"), _f32(k, "k"),
                                     _f32(v, "v"), _f32(g, "g"), _f32(beta, "beta"),
                                     _f32(o, "o", True), n, M, vh, kh, kd, vd)
        _check(rc, "ref_gdn_step_m")

    def slab(self, n_units, dims, hist_floats=0):
        return Slab(self, n_units, dims, hist_floats)

    def conv_push(self, hist, raw, conv_dim, ck):
        self.lib.ref_conv_push(_f32(hist, "hist", True), _f32(raw, "raw"), conv_dim, ck)

    def gdn_frontend(self, x, Wa, Wb, A_log, dt_bias, xc_raw, hist, conv_w,
                     q, k, v, g, beta, dims, ck=4):
        """Front end for B rows; x [B][dim], outputs per row (see gdn_oracle.h)."""
        vh, kh, kd, vd = dims
        B, dim = x.shape
        conv_dim = xc_raw.shape[-1]
        rc = self.lib.ref_gdn_frontend(
            _f32(x, "x"), _f32(Wa, "Wa"), _f32(Wb, "Wb"), _f32(A_log, "A_log"),
            _f32(dt_bias, "dt_bias"), _f32(xc_raw, "xc_raw"), _f32(hist, "hist", True),
            _f32(conv_w, "conv_w"), _f32(q, "q", True), _f32(k, "k", True),
            _f32(v, "v", True), _f32(g, "g", True), _f32(beta, "beta", True),
            B, dim, conv_dim, ck, vh, kh, kd, vd)
        _check(rc, "ref_gdn_frontend")

    def gdn_frontend_m(self, x, Wa, Wb, A_log, dt_bias, xc_raw, hist, conv_w,
                       q, k, v, g, beta, dims, ck=4):
        """M draft rows: x [M][B][dim], xc_raw [M][B][conv_dim], outputs [M][B][...]."""
        vh, kh, kd, vd = dims
        M, B, dim = x.shape
        conv_dim = xc_raw.shape[-1]
        rc = self.lib.ref_gdn_frontend_m(
            _f32(x, "x"), _f32(Wa, "Wa"), _f32(Wb, "Wb"), _f32(A_log, "A_log"),
            _f32(dt_bias, "dt_bias"), _f32(xc_raw, "xc_raw"), _f32(hist, "hist", True),
            _f32(conv_w, "conv_w"), _f32(q, "q", True), _f32(k, "k", True),
            _f32(v, "v", True), _f32(g, "g", True), _f32(beta, "beta", True),
            B, M, dim, conv_dim, ck, vh, kh, kd, vd)
        _check(rc, "ref_gdn_frontend_m")

    def gated_norm(self, o, z, w, eps, out):
        """Gated RMSNorm over the last axis (vd) of o, z -> out."""
        vd = o.shape[-1]
        rows = o.size // vd
        rc = self.lib.ref_gdn_gated_norm(_f32(o, "o"), _f32(z, "z"), _f32(w, "w"), float(eps),
                                         _f32(out, "out", True), rows, vd)
        _check(rc, "ref_gdn_gated_norm")

    def proj(self, x, W, y):
        """y [rows][R] = x [rows][C] . W [R][C]^T, left folds over C."""
        R, Cc = W.shape
        rows = x.size // Cc
        if x.size != rows * Cc or y.size != rows * R:
            raise ValueError("proj: shapes of x, W, y do not agree")
        rc = self.lib.ref_gdn_proj(_f32(x, "x"), _f32(W, "W"), _f32(y, "y", True), rows, R, Cc)
        _check(rc, "ref_gdn_proj")

    def half_to_float(self, h):
        """binary16 bit patterns (uint16 array) -> float32 values."""
        h = np.ascontiguousarray(h, dtype=np.uint16)
        f = np.zeros(h.shape, np.float32)
        self.lib.ref_half_to_float(h.ctypes.data_as(C.c_void_p), f.ctypes.data_as(C.c_void_p),
                                   h.size)
        return f

    def proj_q4(self, x, q, scale, y):
        """y [rows][R] = x . W^T with W decoded from q [R][C/2] (uint8) and
        scale [R][C/32] (binary16 bit patterns, uint16)."""
        R = q.shape[0]
        Cc = 2 * q.shape[1]
        rows = x.size // Cc
        for a, t, nm in ((q, np.uint8, "q"), (scale, np.uint16, "scale")):
            if a.dtype != t or not a.flags.c_contiguous:
                raise TypeError(f"{nm}: need a C-contiguous {t.__name__} array")
        if scale.shape != (R, Cc // 32) or x.size != rows * Cc or y.size != rows * R:
            raise ValueError("proj_q4: shapes of x, q, scale, y do not agree")
        rc = self.lib.ref_gdn_proj_q4(_f32(x, "x"), q.ctypes.data_as(C.c_void_p),
                                      scale.ctypes.data_as(C.c_void_p), _f32(y, "y", True),
                                      rows, R, Cc)
        _check(rc, "ref_gdn_proj_q4")

    def gdn_step64(self, S, q, k, v, g, beta, o, dims):
        """Double-precision brute-force step (tiny shapes, kd, vd <= 16)."""
        vh, kh, kd, vd = dims
        n = S.size // (vh * kd * vd)
        rc = self.lib.ref64_gdn_step(_f64(S, "S"), _f64(q, "q"), _f64(k, "k"),
                                     _f64(v, "v"), _f64(g, "g"), _f64(beta, "beta"),
                                     _f64(o, "o"), n, vh, kh, kd, vd)
        _check(rc, "ref64_gdn_step")


class Slab:
    """Host snapshot slab of the oracle (mark / one-shot rollback)."""

    def __init__(self, orc, n_units, dims, hist_floats=0):
        vh, kh, kd, vd = dims
        self.orc = orc
        self.S_snap = np.zeros(n_units * vh * kd * vd, np.float32)
        self.hist_snap = np.zeros(max(n_units * hist_floats, 1), np.float32)
        self.s = RefSlab(self.S_snap.ctypes.data, self.hist_snap.ctypes.data,
                         n_units, hist_floats, vh, kh, kd, vd, 0)

    @property
    def armed(self):
        return bool(self.s.armed)

    def mark(self, S, hist=None):
        rc = self.orc.lib.ref_gdn_mark(C.byref(self.s), _f32(S, "S"), _opt(hist, "hist"))
        _check(rc, "ref_gdn_mark")

    def rollback(self, S, hist, inputs, M, accepted, xc_raw=None, conv_dim=0, ck=4):
        """inputs: dict q, k, v, g, beta laid out [M][N][...]."""
        acc = np.ascontiguousarray(accepted, dtype=np.int32)
        rc = self.orc.lib.ref_gdn_rollback(
            C.byref(self.s), _f32(S, "S", True), _opt(hist, "hist"),
            _opt(inputs.get("q"), "q"), _opt(inputs.get("k"), "k"),
            _opt(inputs.get("v"), "v"), _opt(inputs.get("g"), "g"),
            _opt(inputs.get("beta"), "beta"), _opt(xc_raw, "xc_raw"),
            conv_dim, ck, M, acc.ctypes.data_as(C.c_void_p))
        _check(rc, "ref_gdn_rollback")


_default = None


def load() -> Oracle:
    """The oracle built from ``gdn_oracle.c`` (compiled on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH) or (
                os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC)):
            build()
        _default = Oracle(LIB_PATH)
    return _default
