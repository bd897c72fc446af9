"""Planted mistakes in the oracle must be caught by its pins.

Each case copies ``oracle/gdn_oracle.c`` into a temporary directory, plants
one plausible mistake (a dropped term, a flipped sign, a wrong index, a
transposed operand, a swapped input), compiles it with the oracle's own flags
and runs every pin against it.  At least one pin has to fail, otherwise the
pins would not be able to tell that oracle from the correct one.  Runs on the
CPU only.
"""
import os
import shutil

import pytest

import oracle
from tests import test_oracle_pins as pins

MUTANTS = [
    ("delta sign", "delta[c] = (vvec[c] - kread[c]) * b;", "delta[c] = (vvec[c] + kread[c]) * b;"),
    ("beta dropped", "delta[c] = (vvec[c] - kread[c]) * b;", "delta[c] = (vvec[c] - kread[c]);"),
    ("decay dropped", "st[(size_t)r * vd + c] = st[(size_t)r * vd + c] * decay;",
     "st[(size_t)r * vd + c] = st[(size_t)r * vd + c] * 1.0f;"),
    ("key read-out before decay",
     "kread[c] = kread[c] + st[(size_t)r * vd + c] * kvec[r];",
     "kread[c] = kread[c] + st[(size_t)r * vd + c] / (decay + 1e-30f) * (decay != 0.0f) * kvec[r];"),
    ("output from the old state", "out[c] = out[c] + st[(size_t)r * vd + c] * qvec[r];",
     "out[c] = out[c] + (st[(size_t)r * vd + c] - kvec[r] * delta[c]) * qvec[r];"),
    ("output reads k instead of q", "out[c] = out[c] + st[(size_t)r * vd + c] * qvec[r];",
     "out[c] = out[c] + st[(size_t)r * vd + c] * kvec[r];"),
    ("rank-1 update uses q",
     "st[(size_t)r * vd + c] = st[(size_t)r * vd + c] + kvec[r] * delta[c];",
     "st[(size_t)r * vd + c] = st[(size_t)r * vd + c] + qvec[r] * delta[c];"),
    ("head mapping modulo", "const int key = i / group;", "const int key = i % kh;"),
    ("transposed state index", "st[(size_t)r * vd + c]", "st[(size_t)c * kd + r]"),
    ("gate not exponentiated", "expf(gu[i]), bu[i]", "gu[i], bu[i]"),
    ("unit offset of g", "g + (size_t)u * vh, beta + (size_t)u * vh,",
     "g, beta + (size_t)u * vh,"),
    ("step_m row stride", "g + m * ng, beta + m * ng", "g, beta + m * ng"),
    ("rollback restores nothing", "memcpy(S, slab->S_snap, (size_t)N * per_s * sizeof(float));", ""),
    ("rollback replays one step short", "for (int m = 0; m < accepted[u]; m++) {",
     "for (int m = 0; m + 1 < accepted[u]; m++) {"),
    ("rollback stays armed", "slab->armed = 0;", ""),
    ("history newest slot", "memcpy(hist + (size_t)(frames - 1) * conv_dim, raw, fb);",
     "memcpy(hist, raw, fb);"),
    ("history not shifted", "memmove(hist, hist + conv_dim, (size_t)(frames - 1) * fb);", ""),
    ("beta from a", "beta[(size_t)b * vh + r] = 1.0f / (1.0f + expf(-acc_b));",
     "beta[(size_t)b * vh + r] = 1.0f / (1.0f + expf(-acc_a));"),
    ("beta sign", "1.0f / (1.0f + expf(-acc_b))", "1.0f / (1.0f + expf(acc_b))"),
    ("gate sign", "return -expf(A_log) * softplus;", "return expf(A_log) * softplus;"),
    ("gate ignores A_log", "return -expf(A_log) * softplus;", "return -softplus;"),
    ("dt_bias dropped", "const float z = a + dt_bias;", "const float z = a;"),
    ("low softplus branch", "softplus = expf(z);", "softplus = 0.0f;"),
    ("high softplus branch", "if (z > 20.0f)\n        softplus = z;",
     "if (z > 20.0f)\n        softplus = 20.0f;"),
    ("conv taps reversed", "y = y + conv_w[(size_t)ch * ck + j] * frames[j][ch];",
     "y = y + conv_w[(size_t)ch * ck + (ck - 1 - j)] * frames[j][ch];"),
    ("conv current tap dropped", "for (int j = 0; j < ck; j++)\n                y = y + conv_w",
     "for (int j = 0; j + 1 < ck; j++)\n                y = y + conv_w"),
    ("silu dropped", "out[ch] = y / (1.0f + expf(-y));", "out[ch] = y;"),
    ("split k offset", "memcpy(kb, out + qk_w,", "memcpy(kb, out,"),
    ("split v offset", "out + 2 * qk_w, (size_t)vh * vd", "out + qk_w, (size_t)vh * vd"),
    ("norm epsilon dropped", "1.0f / sqrtf(ssq + 1e-6f)", "1.0f / sqrtf(ssq)"),
    ("q scale dropped", "qh[j] = (qh[j] * iq) * q_scale;", "qh[j] = qh[j] * iq;"),
    ("k normalised with q's norm", "kk[j] = kk[j] * ik;", "kk[j] = kk[j] * iq;"),
    ("gated norm over the sum", "1.0f / sqrtf(ss / (float)vd + eps)", "1.0f / sqrtf(ss + eps)"),
    ("gated norm eps outside the root", "1.0f / sqrtf(ss / (float)vd + eps)",
     "1.0f / (sqrtf(ss / (float)vd) + eps)"),
    ("gated norm without the root", "1.0f / sqrtf(ss / (float)vd + eps)",
     "1.0f / (ss / (float)vd + eps)"),
    ("gate sigmoid instead of silu", "const float sz = zrow[c] / (1.0f + expf(-zrow[c]));",
     "const float sz = 1.0f / (1.0f + expf(-zrow[c]));"),
    ("norm weight dropped", "out[(size_t)r * vd + c] = ((orow[c] * rinv) * w[c]) * sz;",
     "out[(size_t)r * vd + c] = (orow[c] * rinv) * sz;"),
    ("projection weight transposed", "acc = acc + wo[c] * xr[c];",
     "acc = acc + W[(size_t)c * R + o] * xr[c];"),
    ("projection last term dropped", "for (int c = 0; c < C; c++)\n                acc = acc + wo[c]",
     "for (int c = 0; c + 1 < C; c++)\n                acc = acc + wo[c]"),
    ("projection x row stride", "const float *xr = x + (size_t)r * C;", "const float *xr = x;"),
    ("projection output transposed", "y[(size_t)r * R + o] = acc;",
     "y[(size_t)o * rows + r] = acc;"),
    ("projection folds in double", "float acc = 0.0f;\n            for (int c = 0; c < C; c++)",
     "double acc = 0.0;\n            for (int c = 0; c < C; c++)"),
    ("q4 nibble order swapped", "(c & 1) ? (qo[c / 2] >> 4) : (qo[c / 2] & 0x0f)",
     "(c & 1) ? (qo[c / 2] & 0x0f) : (qo[c / 2] >> 4)"),
    ("q4 nibbles unsigned", "const int n = (nib ^ 8) - 8;", "const int n = nib;"),
    ("q4 scale block of 64", "half_to_float(so[c / 32])", "half_to_float(so[c / 64])"),
    ("half exponent bias", "ldexpf((float)(1024 + f), e - 25)", "ldexpf((float)(1024 + f), e - 24)"),
    ("half subnormals flushed", "mag = ldexpf((float)f, -24);", "mag = 0.0f;"),
    ("half sign dropped", "return (h & 0x8000) ? -mag : mag;", "return mag;"),
]


def _run_pins(orc):
    failed = []
    for pin in pins.PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    return failed


@pytest.fixture(scope="module")
def srcdir(tmp_path_factory):
    d = tmp_path_factory.mktemp("mutants")
    shutil.copy(os.path.join(os.path.dirname(oracle.SRC), "gdn_oracle.h"), d)
    return d


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(srcdir, name, old, new):
    src = open(oracle.SRC).read()
    assert old in src, f"mutation site not found: {old!r}"
    mutated = src.replace(old, new)
    tag = "".join(c if c.isalnum() else "_" for c in name)
    c_path = os.path.join(srcdir, f"m_{tag}.c")
    with open(c_path, "w") as f:
        f.write(mutated)
    so = oracle.build(src=c_path, out=os.path.join(srcdir, f"m_{tag}.so"))
    failed = _run_pins(oracle.Oracle(so))
    assert failed, f"no pin caught the planted mistake '{name}'"


def test_unmutated_copy_passes(srcdir):
    c_path = os.path.join(srcdir, "clean.c")
    shutil.copy(oracle.SRC, c_path)
    so = oracle.build(src=c_path, out=os.path.join(srcdir, "clean.so"))
    assert _run_pins(oracle.Oracle(so)) == []
