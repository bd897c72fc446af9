"""Python binding of the MI355X GDN recurrent-step library (``libgdn_mi355x.so``).

Argument marshalling only: every function checks that its torch tensors are
fp32 (the 4-bit weights: uint8 values and binary16 scales), contiguous and on
a HIP device, derives the sizes from their shapes and calls the C ABI of
``include/gdn.h`` with raw device pointers and the current HIP stream.  All arithmetic runs in the library's gfx950 kernels; there is no
fallback of any kind, and importing this package fails loudly when the
library has not been built (``python -m gated_deltanet_recurrent_amd.build``).

Operator: "Kestrel_VLLM #24: GDN linear attention on GPU", section 4 and
Fig. 1 caption (decay, key read-out, delta, rank-1 update, query read-out with
the updated state); M-step and mark/rollback: "Kestrel_VLLM #34: batched M
rows", sections 3.6 and 3.7; front end: "Kestrel_VLLM #27: register residency
and fused launch", section 4.2, and "#24", section 3; dense projections:
"#24", Fig. 1 caption, steps 1 and 7, and "#34", section 3.6; their 4-bit
weights: "#24", sections 8 and 12.

Every tensor's element count is checked against the sizes passed with it,
because the C ABI receives raw pointers and cannot check them itself.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn_mi355x.so")

GDN_OK, GDN_EINVAL, GDN_EUNSUPPORTED, GDN_ESTATE, GDN_EDEVICE = 0, -1, -2, -3, -4

# Every exported symbol of include/gdn.h.
EXPORTS = ("gdn_strerror", "gdn_step", "gdn_step_m", "gdn_step_gated", "gdn_slab_bytes",
           "gdn_slab_init", "gdn_mark_step_m", "gdn_verify_m", "gdn_commit",
           "gdn_frontend_verify_m",
           "gdn_mark", "gdn_rollback", "gdn_frontend", "gdn_frontend_m", "gdn_stream_copy",
           "gdn_proj", "gdn_proj_pack", "gdn_verify_m_gated", "gdn_proj_q4_bytes",
           "gdn_proj_q4_pack", "gdn_proj_q4", "gdn_stream_read", "gdn_stream_read_words",
           "gdn_rollback_static", "gdn_commit_verify_m")


class GdnError(RuntimeError):
    def __init__(self, rc, what):
        self.rc = rc
        super().__init__(f"{what}: {lib().gdn_strerror(rc).decode()} (rc={rc})")


class gdn_slab(C.Structure):
    _fields_ = [("dev", C.c_void_p), ("bytes", C.c_int64), ("n_units", C.c_int64),
                ("hist_floats", C.c_int64), ("vh", C.c_int32), ("kh", C.c_int32),
                ("kd", C.c_int32), ("vd", C.c_int32), ("armed", C.c_int32),
                ("magic", C.c_int32)]


_lib = None


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m gated_deltanet_recurrent_amd.build` (there is no fallback path)")
    L = C.CDLL(LIB_PATH)
    P, I32, I64 = C.c_void_p, C.c_int32, C.c_int64
    L.gdn_strerror.argtypes = [C.c_int]
    L.gdn_strerror.restype = C.c_char_p
    L.gdn_step.argtypes = [P] * 7 + [I64, I32, I32, I32, I32, P]
    L.gdn_step_m.argtypes = [P] * 7 + [I64, I32, I32, I32, I32, I32, P]
    L.gdn_step_gated.argtypes = [P] * 8 + [C.c_float, P, I64, I32, I32, I32, I32, I32, P]
    L.gdn_slab_bytes.argtypes = [I64, I32, I32, I32, I32, I64]
    L.gdn_slab_bytes.restype = I64
    L.gdn_slab_init.argtypes = [C.POINTER(gdn_slab), P, I64, I64, I32, I32, I32, I32, I64]
    L.gdn_mark.argtypes = [C.POINTER(gdn_slab), P, P, P]
    L.gdn_mark_step_m.argtypes = [C.POINTER(gdn_slab)] + [P] * 8 + [I64, I32, I32, I32, I32, I32, P]
    L.gdn_rollback.argtypes = [C.POINTER(gdn_slab)] + [P] * 8 + [I32, I32, I32, P, P]
    L.gdn_rollback_static.argtypes = L.gdn_rollback.argtypes
    L.gdn_frontend.argtypes = [P] * 13 + [I32] * 8 + [P]
    L.gdn_frontend_m.argtypes = [P] * 13 + [I32] * 9 + [P]
    L.gdn_stream_copy.argtypes = [P, P, I64, P]
    L.gdn_stream_read.argtypes = [P, I64, P, P]
    L.gdn_stream_read_words.argtypes = [I64]
    L.gdn_stream_read_words.restype = I64
    L.gdn_verify_m.argtypes = [P] * 7 + [I64, I32, I32, I32, I32, I32, P]
    L.gdn_commit.argtypes = [P] * 8 + [I32, I32, I64, I32, I32, I32, I32, I32, P, P, P]
    L.gdn_commit_verify_m.argtypes = ([P] * 8 + [I32, I32, I64, I32, P, P] + [P] * 6
                                      + [I32, I32, I32, I32, I32, P])
    L.gdn_frontend_verify_m.argtypes = [P] * 13 + [I32] * 9 + [P]
    L.gdn_proj.argtypes = [P, I64, I32, P, I32, P, P, I32, P, P]
    L.gdn_proj_pack.argtypes = [P, P, I32, I32, P]
    L.gdn_verify_m_gated.argtypes = [P] * 8 + [C.c_float, P, I64, I32, I32, I32, I32, I32, P]
    L.gdn_proj_q4_bytes.argtypes = [I32, I32]
    L.gdn_proj_q4_bytes.restype = I64
    L.gdn_proj_q4_pack.argtypes = [P, P, P, I32, I32, P]
    L.gdn_proj_q4.argtypes = [P, I64, I32, P, I32, P, P, I32, P, P]
    for f in ("gdn_step", "gdn_step_m", "gdn_step_gated", "gdn_slab_init", "gdn_mark_step_m", "gdn_mark", "gdn_rollback",
              "gdn_rollback_static", "gdn_frontend", "gdn_frontend_m", "gdn_stream_copy", "gdn_stream_read",
              "gdn_verify_m",
              "gdn_commit", "gdn_commit_verify_m", "gdn_frontend_verify_m", "gdn_proj",
              "gdn_proj_pack",
              "gdn_verify_m_gated", "gdn_proj_q4_pack", "gdn_proj_q4"):
        getattr(L, f).restype = C.c_int
    _lib = L
    return L


def _dev(t, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be on a HIP device, got {t.device}")
    if t.dtype != torch.float32:
        raise TypeError(f"{name}: must be float32, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return C.c_void_p(t.data_ptr())


def _sized(t, n, name):
    """_dev plus an element-count check: the C ABI takes raw pointers, so a
    tensor smaller than the sizes passed with it would be read or written
    out of bounds on the device."""
    if t is None:
        return None
    p = _dev(t, name)
    if t.numel() != n:
        raise ValueError(f"{name}: has {t.numel()} elements, the call needs {n}")
    return p


def _rows(S, q, k, v, g, beta, M, o=None, o_name="o"):
    """Pointers of the per-row inputs of M steps over the units of S, each
    size-checked: q, k [M][N][kh][kd]; v, o [M][N][vh][vd]; g, beta [M][N][vh]."""
    N, vh, kd, vd = S.shape
    kh = q.shape[-2]
    qk = M * N * kh * kd
    return [_sized(q, qk, "q"), _sized(k, qk, "k"), _sized(v, M * N * vh * vd, "v"),
            _sized(g, M * N * vh, "g"), _sized(beta, M * N * vh, "beta")] + (
        [_sized(o, M * N * vh * vd, o_name)] if o is not None else [])


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _check(rc, what):
    if rc != GDN_OK:
        raise GdnError(rc, what)


def _state_dims(S, q, v):
    """(n_units, vh, kh, kd, vd) from S [N][vh][kd][vd], q [.., N, kh, kd]."""
    if S.dim() != 4 or q.dim() < 3:
        raise ValueError("S must be [N][vh][kd][vd] and q [..][N][kh][kd]")
    N, vh, kd, vd = S.shape
    kh = q.shape[-2]
    return N, vh, kh, kd, vd


def step(S, q, k, v, g, beta, o=None, stream=None):
    """One decode step for every unit (gdn_step).  S [N][vh][kd][vd] advances
    in place; returns o [N][vh][vd]."""
    N, vh, kh, kd, vd = _state_dims(S, q, v)
    if o is None:
        o = torch.empty((N, vh, vd), dtype=torch.float32, device=S.device)
    _check(lib().gdn_step(_dev(S, "S"), *_rows(S, q, k, v, g, beta, 1, o), N, vh, kh, kd,
                          vd, _stream(stream)), "gdn_step")
    return o


def step_m(S, q, k, v, g, beta, o=None, stream=None):
    """M sequential steps (gdn_step_m); q, k [M][N][kh][kd], v [M][N][vh][vd],
    g, beta [M][N][vh].  Returns o [M][N][vh][vd]."""
    N, vh, kh, kd, vd = _state_dims(S, q, v)
    M = q.shape[0]
    if o is None:
        o = torch.empty((M, N, vh, vd), dtype=torch.float32, device=S.device)
    _check(lib().gdn_step_m(_dev(S, "S"), *_rows(S, q, k, v, g, beta, M, o), N, M, vh, kh,
                            kd, vd, _stream(stream)), "gdn_step_m")
    return o


def step_gated(S, q, k, v, g, beta, z, norm_w, eps=1e-6, out=None, stream=None):
    """M steps with the gated RMSNorm fused on the output (gdn_step_gated).
    q, k [M][N][kh][kd]; v, z [M][N][vh][vd]; g, beta [M][N][vh]; norm_w
    [vd].  Returns out [M][N][vh][vd]."""
    N, vh, kh, kd, vd = _state_dims(S, q, v)
    M = q.shape[0]
    if out is None:
        out = torch.empty((M, N, vh, vd), dtype=torch.float32, device=S.device)
    _check(lib().gdn_step_gated(_dev(S, "S"), *_rows(S, q, k, v, g, beta, M),
                                _sized(z, M * N * vh * vd, "z"), _sized(norm_w, vd, "norm_w"),
                                float(eps), _sized(out, M * N * vh * vd, "out"), N, M, vh,
                                kh, kd, vd, _stream(stream)), "gdn_step_gated")
    return out


def slab_bytes(n_units, dims, hist_floats_per_unit=0):
    vh, kh, kd, vd = dims
    nb = lib().gdn_slab_bytes(n_units, vh, kh, kd, vd, hist_floats_per_unit)
    if nb < 0:
        raise GdnError(int(nb), "gdn_slab_bytes")
    return int(nb)


class Slab:
    """Snapshot slab: host struct + device buffer (a torch uint8 tensor)."""

    def __init__(self, n_units, dims, hist_floats_per_unit=0, device="cuda"):
        vh, kh, kd, vd = dims
        nb = slab_bytes(n_units, dims, hist_floats_per_unit)
        self.buf = torch.empty(nb, dtype=torch.uint8, device=device)
        self.s = gdn_slab()
        _check(lib().gdn_slab_init(C.byref(self.s), C.c_void_p(self.buf.data_ptr()), nb,
                                   n_units, vh, kh, kd, vd, hist_floats_per_unit),
               "gdn_slab_init")

    @property
    def armed(self):
        return int(self.s.armed)

    def _state_sizes(self):
        sl = self.s
        return sl.n_units * sl.vh * sl.kd * sl.vd, sl.n_units * sl.hist_floats

    def _hist(self, hist):
        # a slab without a history area: the C ABI refuses any hist (GDN_ESTATE)
        # before anything is enqueued, so there is no size to check
        nh = self.s.n_units * self.s.hist_floats
        return _sized(hist, nh, "hist") if nh else _dev(hist, "hist")

    def mark(self, S, hist=None, stream=None):
        ns = self._state_sizes()[0]
        _check(lib().gdn_mark(C.byref(self.s), _sized(S, ns, "S"), self._hist(hist),
                              _stream(stream)), "gdn_mark")

    def mark_step_m(self, S, q, k, v, g, beta, hist=None, o=None, stream=None):
        """gdn_mark_step_m: mark S (and hist) and run M steps, reading S once.
        Returns o [M][N][vh][vd]."""
        N, vh, kh, kd, vd = _state_dims(S, q, v)
        M = q.shape[0]
        if o is None:
            o = torch.empty((M, N, vh, vd), dtype=torch.float32, device=S.device)
        ns = self._state_sizes()[0]
        _check(lib().gdn_mark_step_m(C.byref(self.s), _sized(S, ns, "S"),
                                     self._hist(hist),
                                     *_rows(S, q, k, v, g, beta, M, o), N, M, vh, kh, kd, vd,
                                     _stream(stream)), "gdn_mark_step_m")
        return o

    def rollback(self, S, accepted, q=None, k=None, v=None, g=None, beta=None, hist=None,
                 xc_raw=None, M=None, stream=None, static_counts=False):
        """accepted: host int32 per unit (list, numpy or CPU tensor).
        static_counts: stage the counts in the library's own area
        (gdn_rollback_static) instead of the slab's."""
        acc = torch.as_tensor(accepted, dtype=torch.int32).contiguous().cpu()
        if acc.numel() != self.s.n_units:
            raise ValueError("accepted must hold one entry per unit")
        if M is None:
            M = q.shape[0] if q is not None else 1
        conv_dim = xc_raw.shape[-1] if xc_raw is not None else (
            hist.shape[-1] if hist is not None else 0)
        ns = self._state_sizes()[0]
        rows = _rows(S, q, k, v, g, beta, M) if q is not None else [None] * 5
        fn = lib().gdn_rollback_static if static_counts else lib().gdn_rollback
        _check(fn(C.byref(self.s), _sized(S, ns, "S"), self._hist(hist), *rows,
                  _sized(xc_raw, M * self.s.n_units * conv_dim, "xc_raw"),
                  conv_dim, 4, M, C.c_void_p(acc.data_ptr()), _stream(stream)),
               "gdn_rollback_static" if static_counts else "gdn_rollback")


def _fe_args(x, Wa, Wb, A_log, dt_bias, xc_raw, hist, conv_w, out, dims, M, B, dim):
    """Size-checked pointers of a front-end call over M rows of B units."""
    vh, kh, kd, vd = dims
    conv_dim = xc_raw.shape[-1]
    ck = conv_w.shape[-1]
    return [_sized(x, M * B * dim, "x"), _sized(Wa, vh * dim, "Wa"), _sized(Wb, vh * dim, "Wb"),
            _sized(A_log, vh, "A_log"), _sized(dt_bias, vh, "dt_bias"),
            _sized(xc_raw, M * B * conv_dim, "xc_raw"),
            _sized(hist, B * (ck - 1) * conv_dim, "hist"),
            _sized(conv_w, conv_dim * ck, "conv_w"),
            _sized(out["q"], M * B * kh * kd, "q"), _sized(out["k"], M * B * kh * kd, "k"),
            _sized(out["v"], M * B * vh * vd, "v"), _sized(out["g"], M * B * vh, "g"),
            _sized(out["beta"], M * B * vh, "beta")]


def frontend(x, Wa, Wb, A_log, dt_bias, xc_raw, hist, conv_w, dims, out=None, stream=None):
    """Front end for B rows (gdn_frontend).  Returns dict q, k, v, g, beta."""
    vh, kh, kd, vd = dims
    B, dim = x.shape
    conv_dim = xc_raw.shape[-1]
    ck = conv_w.shape[-1]
    dev = x.device
    if out is None:
        out = dict(q=torch.empty((B, kh, kd), dtype=torch.float32, device=dev),
                   k=torch.empty((B, kh, kd), dtype=torch.float32, device=dev),
                   v=torch.empty((B, vh, vd), dtype=torch.float32, device=dev),
                   g=torch.empty((B, vh), dtype=torch.float32, device=dev),
                   beta=torch.empty((B, vh), dtype=torch.float32, device=dev))
    _check(lib().gdn_frontend(
        *_fe_args(x, Wa, Wb, A_log, dt_bias, xc_raw, hist, conv_w, out, dims, 1, B, dim),
        B, dim, conv_dim, ck, vh, kh, kd, vd, _stream(stream)), "gdn_frontend")
    return out


def frontend_m(x, Wa, Wb, A_log, dt_bias, xc_raw, hist, conv_w, dims, out=None, stream=None):
    """Front end for M draft rows (gdn_frontend_m): x [M][B][dim], xc_raw
    [M][B][conv_dim]; the history advances M frames.  Returns dict q, k, v, g,
    beta laid out [M][B][...] (the rows gdn_step_m takes)."""
    vh, kh, kd, vd = dims
    M, B, dim = x.shape
    conv_dim = xc_raw.shape[-1]
    ck = conv_w.shape[-1]
    dev = x.device
    if out is None:
        out = dict(q=torch.empty((M, B, kh, kd), dtype=torch.float32, device=dev),
                   k=torch.empty((M, B, kh, kd), dtype=torch.float32, device=dev),
                   v=torch.empty((M, B, vh, vd), dtype=torch.float32, device=dev),
                   g=torch.empty((M, B, vh), dtype=torch.float32, device=dev),
                   beta=torch.empty((M, B, vh), dtype=torch.float32, device=dev))
    _check(lib().gdn_frontend_m(
        *_fe_args(x, Wa, Wb, A_log, dt_bias, xc_raw, hist, conv_w, out, dims, M, B, dim),
        B, M, dim, conv_dim, ck, vh, kh, kd, vd, _stream(stream)), "gdn_frontend_m")
    return out


def verify_m(S, q, k, v, g, beta, o=None, stream=None):
    """Outputs of M draft rows without advancing S (gdn_verify_m)."""
    N, vh, kh, kd, vd = _state_dims(S, q, v)
    M = q.shape[0]
    if o is None:
        o = torch.empty((M, N, vh, vd), dtype=torch.float32, device=S.device)
    _check(lib().gdn_verify_m(_dev(S, "S"), *_rows(S, q, k, v, g, beta, M, o), N, M, vh, kh,
                              kd, vd, _stream(stream)), "gdn_verify_m")
    return o


def _int32_dev(t, name, n):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype != torch.int32 \
            or not t.is_contiguous():
        raise TypeError(f"{name}: need a contiguous int32 tensor on a HIP device")
    if t.numel() != n:
        raise ValueError(f"{name}: has {t.numel()} elements, the call needs {n}")
    return C.c_void_p(t.data_ptr())


def verify_m_gated(S, q, k, v, g, beta, z, norm_w, eps=1e-6, out=None, stream=None):
    """Gated outputs of M draft rows without advancing S (gdn_verify_m_gated).
    z [M][N][vh][vd]; norm_w [vd].  Returns out [M][N][vh][vd]."""
    N, vh, kh, kd, vd = _state_dims(S, q, v)
    M = q.shape[0]
    if out is None:
        out = torch.empty((M, N, vh, vd), dtype=torch.float32, device=S.device)
    _check(lib().gdn_verify_m_gated(_dev(S, "S"), *_rows(S, q, k, v, g, beta, M),
                                    _sized(z, M * N * vh * vd, "z"),
                                    _sized(norm_w, vd, "norm_w"), float(eps),
                                    _sized(out, M * N * vh * vd, "out"), N, M,
                                    vh, kh, kd, vd, _stream(stream)), "gdn_verify_m_gated")
    return out


def commit(S, accepted, q, k, v, g, beta, hist=None, xc_raw=None, status=None, stream=None):
    """Apply the accepted prefix of the M rows given to verify_m (gdn_commit).
    accepted: int32 device tensor [N]; status: int32 device tensor [1] or
    None (set to 1 when an entry is out of range)."""
    N, vh, kh, kd, vd = _state_dims(S, q, v)
    M = q.shape[0]
    conv_dim = xc_raw.shape[-1] if xc_raw is not None else 0
    _check(lib().gdn_commit(_dev(S, "S"), _sized(hist, N * 3 * conv_dim, "hist"),
                            *_rows(S, q, k, v, g, beta, M),
                            _sized(xc_raw, M * N * conv_dim, "xc_raw"), conv_dim, 4, N, M, vh, kh,
                            kd, vd, _int32_dev(accepted, "accepted", N),
                            _int32_dev(status, "status", 1), _stream(stream)), "gdn_commit")


def commit_verify_m(S, accepted, q, k, v, g, beta, q2, k2, v2, g2, beta2, o=None, hist=None,
                    xc_raw=None, status=None, stream=None):
    """commit (the accepted prefix of the previous rows q..beta [M][N]) and
    then verify_m of the next rows q2..beta2 [M2][N], in one pass over S
    (gdn_commit_verify_m).  Returns o [M2][N][vh][vd]."""
    N, vh, kh, kd, vd = _state_dims(S, q, v)
    M, M2 = q.shape[0], q2.shape[0]
    if o is None:
        o = torch.empty((M2, N, vh, vd), dtype=torch.float32, device=S.device)
    conv_dim = xc_raw.shape[-1] if xc_raw is not None else 0
    _check(lib().gdn_commit_verify_m(
        _dev(S, "S"), _sized(hist, N * 3 * conv_dim, "hist"), *_rows(S, q, k, v, g, beta, M),
        _sized(xc_raw, M * N * conv_dim, "xc_raw"), conv_dim, 4, N, M,
        _int32_dev(accepted, "accepted", N), _int32_dev(status, "status", 1),
        *_rows(S, q2, k2, v2, g2, beta2, M2, o), M2, vh, kh, kd, vd, _stream(stream)),
        "gdn_commit_verify_m")
    return o


def frontend_verify_m(x, Wa, Wb, A_log, dt_bias, xc_raw, hist, conv_w, dims, out=None,
                      stream=None):
    """frontend_m without advancing the history (gdn_frontend_verify_m)."""
    vh, kh, kd, vd = dims
    M, B, dim = x.shape
    conv_dim = xc_raw.shape[-1]
    ck = conv_w.shape[-1]
    dev = x.device
    if out is None:
        out = dict(q=torch.empty((M, B, kh, kd), dtype=torch.float32, device=dev),
                   k=torch.empty((M, B, kh, kd), dtype=torch.float32, device=dev),
                   v=torch.empty((M, B, vh, vd), dtype=torch.float32, device=dev),
                   g=torch.empty((M, B, vh), dtype=torch.float32, device=dev),
                   beta=torch.empty((M, B, vh), dtype=torch.float32, device=dev))
    _check(lib().gdn_frontend_verify_m(
        *_fe_args(x, Wa, Wb, A_log, dt_bias, xc_raw, hist, conv_w, out, dims, M, B, dim),
        B, M, dim, conv_dim, ck, vh, kh, kd, vd, _stream(stream)), "gdn_frontend_verify_m")
    return out


def proj_pack(W, out=None, stream=None):
    """Weights W [R][C] (row-major) in the packed order gdn_proj reads
    (gdn_proj_pack); returns a tensor of the same shape holding that order."""
    if W.dim() != 2:
        raise ValueError("W must be [R][C]")
    if out is None:
        out = torch.empty_like(W)
    _check(lib().gdn_proj_pack(_dev(W, "W"), _dev(out, "Wp"), W.shape[0], W.shape[1],
                               _stream(stream)), "gdn_proj_pack")
    return out


def proj(x, W0, W1=None, y0=None, y1=None, stream=None):
    """Dense projection(s) of the layer (gdn_proj): y0 = x W0^T and, with W1,
    y1 = x W1^T in the same launch.  x [..., C] (leading axes are rows);
    W0, W1: [R][C] weights already packed by proj_pack; outputs [..., R].
    Returns y0, or (y0, y1) when W1 is given."""
    Cc = x.shape[-1]
    lead = tuple(x.shape[:-1])
    rows = x.numel() // Cc if Cc else 0
    for W, nm in ((W0, "W0"), (W1, "W1")):
        if W is not None and (W.dim() != 2 or W.shape[1] != Cc):
            raise ValueError(f"{nm} must be [R][{Cc}]")
    if y0 is None:
        y0 = torch.empty(lead + (W0.shape[0],), dtype=torch.float32, device=x.device)
    if W1 is not None and y1 is None:
        y1 = torch.empty(lead + (W1.shape[0],), dtype=torch.float32, device=x.device)
    if y0.numel() != rows * W0.shape[0] or (W1 is not None and y1.numel() != rows * W1.shape[0]):
        raise ValueError("output sizes do not match rows x R")
    R1 = W1.shape[0] if W1 is not None else 0
    _check(lib().gdn_proj(_dev(x, "x"), rows, Cc, _dev(W0, "W0"), W0.shape[0], _dev(y0, "y0"),
                          _dev(W1, "W1"), R1, _dev(y1, "y1"), _stream(stream)), "gdn_proj")
    return y0 if W1 is None else (y0, y1)


def _dev_bytes(t, name, dtypes):
    """Device pointer of a contiguous tensor of one of the given dtypes."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be on a HIP device, got {t.device}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: must be one of {dtypes}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return C.c_void_p(t.data_ptr())


def proj_q4_bytes(R, C_):
    """Bytes of a packed 4-bit [R][C] weight matrix (gdn_proj_q4_bytes)."""
    n = lib().gdn_proj_q4_bytes(R, C_)
    if n < 0:
        raise GdnError(GDN_EUNSUPPORTED, f"gdn_proj_q4_bytes: R={R}, C={C_} not supported")
    return n


def proj_q4_pack(q, scale, out=None, stream=None):
    """4-bit weights in the packed order gdn_proj_q4 reads (gdn_proj_q4_pack).
    q: uint8 [R][C/2] (element 2i in the low nibble of byte i, two's
    complement); scale: [R][C/32] binary16 (float16, or int16 bit patterns).
    Returns uint8 [R/64][36 C]: one row per group of 64 weight rows."""
    if q.dim() != 2 or scale.dim() != 2:
        raise ValueError("q must be [R][C/2] and scale [R][C/32]")
    R, Cc = q.shape[0], 2 * q.shape[1]
    if tuple(scale.shape) != (R, Cc // 32) or Cc % 32:
        raise ValueError(f"scale must be [{R}][{Cc // 32}] for q of shape {tuple(q.shape)}")
    n = proj_q4_bytes(R, Cc)
    if out is None:
        out = torch.empty((R // 64, 36 * Cc), dtype=torch.uint8, device=q.device)
    if out.numel() != n:
        raise ValueError(f"out must hold {n} bytes")
    _check(lib().gdn_proj_q4_pack(_dev_bytes(q, "q", (torch.uint8,)),
                                  _dev_bytes(scale, "scale", (torch.float16, torch.int16)),
                                  _dev_bytes(out, "Wq", (torch.uint8,)), R, Cc,
                                  _stream(stream)), "gdn_proj_q4_pack")
    return out


def proj_q4(x, Wq0, Wq1=None, y0=None, y1=None, stream=None):
    """proj with 4-bit weights (gdn_proj_q4): Wq0, Wq1 packed by proj_q4_pack
    (uint8 [R/64][36 C]); x [..., C] with 1 to 16 rows.  Returns y0, or
    (y0, y1) when Wq1 is given."""
    Cc = x.shape[-1]
    lead = tuple(x.shape[:-1])
    rows = x.numel() // Cc if Cc else 0
    Rs = []
    for W, nm in ((Wq0, "Wq0"), (Wq1, "Wq1")):
        if W is None:
            Rs.append(0)
            continue
        if W.dim() != 2 or W.shape[1] != 36 * Cc:
            raise ValueError(f"{nm} must be a packed [R/64][{36 * Cc}] uint8 matrix")
        Rs.append(64 * W.shape[0])
    if y0 is None:
        y0 = torch.empty(lead + (Rs[0],), dtype=torch.float32, device=x.device)
    if Wq1 is not None and y1 is None:
        y1 = torch.empty(lead + (Rs[1],), dtype=torch.float32, device=x.device)
    if y0.numel() != rows * Rs[0] or (Wq1 is not None and y1.numel() != rows * Rs[1]):
        raise ValueError("output sizes do not match rows x R")
    _check(lib().gdn_proj_q4(_dev(x, "x"), rows, Cc, _dev_bytes(Wq0, "Wq0", (torch.uint8,)),
                             Rs[0], _dev(y0, "y0"), _dev_bytes(Wq1, "Wq1", (torch.uint8,)), Rs[1],
                             _dev(y1, "y1"), _stream(stream)), "gdn_proj_q4")
    return y0 if Wq1 is None else (y0, y1)


def stream_copy(dst, src, stream=None):
    """128-bit streaming copy (the read+write floor); dst may be src."""
    if dst.numel() != src.numel():
        raise ValueError("dst and src sizes differ")
    _check(lib().gdn_stream_copy(_dev(dst, "dst"), _dev(src, "src"), src.numel(),
                                 _stream(stream)), "gdn_stream_copy")


def stream_read(src, words=None, stream=None):
    """Read-only floor (gdn_stream_read): streams src and returns one uint32
    word per 128 KiB chunk, the XOR of the chunk's 32-bit words (as an int32
    tensor holding the same bits)."""
    n = src.numel()
    nw = int(lib().gdn_stream_read_words(max(n, 1)))
    if words is None:
        words = torch.empty(nw, dtype=torch.int32, device=src.device)
    if words.dtype != torch.int32 or not words.is_contiguous() or words.numel() != nw \
            or words.device.type != "cuda":
        raise ValueError(f"words: need a contiguous int32 HIP tensor of {nw} elements")
    _check(lib().gdn_stream_read(_dev(src, "src"), n, C.c_void_p(words.data_ptr()),
                                 _stream(stream)), "gdn_stream_read")
    return words
