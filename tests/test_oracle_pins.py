"""Pins of the CPU oracle: facts fixed by the operator's definition and by
mathematics, not by the oracle itself.

The operator (value head i, key head i/(vh/kh); "Kestrel_VLLM #24: GDN linear
attention on GPU", section 4 and Fig. 1 caption):
    alpha = exp(g);  S <- alpha S;  kv = S^T k;  tmp = (v - kv) beta;
    S <- S + k tmp^T;  o = S^T q   (with the updated S)
Front end (same page, section 3; "Kestrel_VLLM #27", section 4.2):
    a = Wa x, b = Wb x; g = -exp(A_log) softplus(a + dt_bias); beta = sigmoid(b);
    depthwise causal conv over [history frames..., raw] + SiLU; history keeps
    raw inputs; split q | k | v; per key head L2 norm (q also / sqrt(kd)).

Every pin is a function ``pin_*(orc)`` so that the mutation test can run the
same pins against deliberately broken copies of the oracle.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit

from tests.helpers import assert_close, bits_equal

DIMS_SMALL = [(3, 1, 4, 4), (1, 1, 4, 4), (6, 2, 4, 3), (4, 4, 3, 5)]


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return (x / np.linalg.norm(x, axis=-1, keepdims=True))


def rand_inputs(r, N, dims, M=1, s_std=0.3):
    vh, kh, kd, vd = dims
    S = r.normal(0, s_std, (N, vh, kd, vd)).astype(np.float32)
    q = (_unit(r.normal(size=(M, N, kh, kd))) / np.sqrt(kd)).astype(np.float32)
    k = _unit(r.normal(size=(M, N, kh, kd))).astype(np.float32)
    v = r.normal(size=(M, N, vh, vd)).astype(np.float32)
    g = (-np.logaddexp(0.0, r.normal(size=(M, N, vh)))).astype(np.float32)
    beta = expit(r.normal(size=(M, N, vh))).astype(np.float32)
    return S, dict(q=q, k=k, v=v, g=g, beta=beta)


def row(inp, m):
    return {n: np.ascontiguousarray(a[m]) for n, a in inp.items()}


def step(orc, S, inp, dims):
    vh, kh, kd, vd = dims
    N = S.shape[0]
    o = np.zeros((N, vh, vd), np.float32)
    orc.gdn_step(S, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], o, dims)
    return o


# --------------------------------------------------------------------------
# the step
# --------------------------------------------------------------------------

def pin_brute_force_fp64(orc):
    """Tiny shapes, 5 chained steps: the fp32 column-wise oracle against the
    double-precision re-associated matrix form alpha (I - beta k k^T) S +
    beta k v^T (different formula, different precision).  Non-square kd x vd
    catches transposed operands; vh > kh catches the head mapping."""
    for t, dims in enumerate(DIMS_SMALL):
        r = _rng(100 + t)
        S, inp = rand_inputs(r, 2, dims, M=5)
        S64 = S.astype(np.float64)
        for m in range(5):
            x = row(inp, m)
            o = step(orc, S, x, dims)
            o64 = np.zeros(o.shape, np.float64)
            orc.gdn_step64(S64, *(x[n].astype(np.float64) for n in
                                  ("q", "k", "v", "g", "beta")), o64, dims)
            assert_close(S, S64, f"S {dims} step {m}")
            assert_close(o, o64, f"o {dims} step {m}")


def pin_exact_dyadic(orc):
    """alpha = 1 (g = 0), beta = 1/2, entries k/4 with small k: every fp32
    operation is exact, so the oracle must equal the exact rational value of
    S' = S + beta k (v - S^T k)^T and o = S'^T q, element for element."""
    r = _rng(7)
    dims = (2, 1, 4, 3)
    vh, kh, kd, vd = dims
    S = (r.integers(-4, 5, (1, vh, kd, vd)) / 4).astype(np.float32)
    q = (r.integers(-2, 3, (1, kh, kd)) / 4).astype(np.float32)
    k = (r.integers(-2, 3, (1, kh, kd)) / 4).astype(np.float32)
    v = (r.integers(-4, 5, (1, vh, vd)) / 4).astype(np.float32)
    g = np.zeros((1, vh), np.float32)
    beta = np.full((1, vh), 0.5, np.float32)
    want_S = np.zeros((vh, kd, vd), object)
    want_o = np.zeros((vh, vd), object)
    for i in range(vh):
        Sm = [[Fraction(float(S[0, i, a, c])) for c in range(vd)] for a in range(kd)]
        kk = [Fraction(float(x)) for x in k[0, i // (vh // kh)]]
        qq = [Fraction(float(x)) for x in q[0, i // (vh // kh)]]
        vv = [Fraction(float(x)) for x in v[0, i]]
        b = Fraction(1, 2)
        Stk = [sum(Sm[a][c] * kk[a] for a in range(kd)) for c in range(vd)]
        for a in range(kd):
            for c in range(vd):
                want_S[i, a, c] = Sm[a][c] + b * kk[a] * (vv[c] - Stk[c])
        for c in range(vd):
            want_o[i, c] = sum(want_S[i, a, c] * qq[a] for a in range(kd))
    o = step(orc, S, dict(q=q, k=k, v=v, g=g, beta=beta), dims)
    assert np.array_equal(S[0].astype(np.float64), want_S.astype(np.float64))
    assert np.array_equal(o[0].astype(np.float64), want_o.astype(np.float64))


def pin_delta_rule_invariant(orc):
    """beta = 1, alpha = 1, unit-norm k  =>  S'^T k = v (the delta rule writes
    v under key k): S'^T k = S^T k + (k^T k)(v - S^T k)."""
    dims = (48, 16, 128, 128)
    r = _rng(3)
    S, inp = rand_inputs(r, 2, dims, s_std=0.02)
    inp["g"][:] = 0.0
    inp["beta"][:] = 1.0
    step(orc, S, row(inp, 0), dims)
    k = inp["k"][0].astype(np.float64)
    kfull = np.repeat(k, 3, axis=1)                       # [N][vh][kd]
    Stk = np.einsum("nhab,nha->nhb", S.astype(np.float64), kfull)
    assert_close(Stk, inp["v"][0], "S'^T k vs v", rel=1e-5, floor=1e-5)


def pin_one_hot_key_overwrites_row(orc):
    """alpha = 1, beta = 1, k = e_j: row j of S becomes v (up to one rounding
    of S + (v - S)), other rows are untouched bit for bit, and with q = e_j
    the output is the UPDATED row j, i.e. v, not the old row."""
    dims = (3, 1, 8, 6)
    vh, kh, kd, vd = dims
    r = _rng(11)
    S, inp = rand_inputs(r, 1, dims)
    j = 5
    inp["k"][:] = 0.0
    inp["k"][0, 0, 0, j] = 1.0
    inp["q"][:] = 0.0
    inp["q"][0, 0, 0, j] = 1.0
    inp["g"][:] = 0.0
    inp["beta"][:] = 1.0
    S0 = S.copy()
    o = step(orc, S, row(inp, 0), dims)
    others = [a for a in range(kd) if a != j]
    assert bits_equal(S[:, :, others, :], S0[:, :, others, :])
    assert_close(S[0, :, j, :], inp["v"][0, 0], "row j", rel=2e-7, floor=1e-7)
    assert_close(o[0], inp["v"][0, 0], "o = updated row", rel=2e-7, floor=1e-7)


def pin_reset_gate(orc):
    """g = -inf => alpha = 0 exactly, kv = 0, and S' = fl(k * fl(v * beta))
    bit for bit; o = tmp (k . q)."""
    dims = (6, 2, 8, 8)
    vh, kh, kd, vd = dims
    r = _rng(5)
    S, inp = rand_inputs(r, 3, dims)
    inp["g"][:] = -np.inf
    o = step(orc, S, row(inp, 0), dims)
    rep = vh // kh
    kf = np.repeat(inp["k"][0], rep, axis=1)              # [N][vh][kd]
    qf = np.repeat(inp["q"][0], rep, axis=1)
    tmp = inp["v"][0] * inp["beta"][0][..., None]         # fp32 multiply
    want = kf[..., :, None] * tmp[..., None, :]           # fp32 multiply
    assert np.array_equal(S, want)
    kq = np.sum(kf.astype(np.float64) * qf, axis=-1)
    assert_close(o, tmp.astype(np.float64) * kq[..., None], "o at reset")


def pin_zero_beta(orc):
    """beta = 0: with g = 0 the state is unchanged bit for bit and o = S^T q
    (a plain matrix-vector product); with general g, S' = exp(g) S."""
    dims = (6, 2, 16, 8)
    vh, kh, kd, vd = dims
    r = _rng(9)
    S, inp = rand_inputs(r, 2, dims)
    inp["beta"][:] = 0.0
    inp["g"][:] = 0.0
    S0 = S.copy()
    o = step(orc, S, row(inp, 0), dims)
    assert bits_equal(S, S0)
    qf = np.repeat(inp["q"][0], vh // kh, axis=1).astype(np.float64)
    assert_close(o, np.einsum("nhab,nha->nhb", S0.astype(np.float64), qf), "S^T q")
    S, inp = rand_inputs(r, 2, dims)
    inp["beta"][:] = 0.0
    S0 = S.copy()
    step(orc, S, row(inp, 0), dims)
    alpha = np.exp(inp["g"][0].astype(np.float64))[..., None, None]
    assert_close(S, alpha * S0, "alpha S", rel=3e-7, floor=1e-30)


def pin_head_mapping(orc):
    """Value head i reads key head i // (vh/kh): perturbing key head j changes
    exactly value heads rep*j .. rep*j + rep - 1."""
    dims = (6, 2, 4, 4)
    vh, kh, kd, vd = dims
    rep = vh // kh
    r = _rng(13)
    S, inp = rand_inputs(r, 1, dims)
    base_S = S.copy()
    o_base = step(orc, base_S, row(inp, 0), dims)
    for j in range(kh):
        pert = {n: a.copy() for n, a in inp.items()}
        pert["k"][0, 0, j] = _unit(pert["k"][0, 0, j][::-1].copy())
        S2 = S.copy()
        o2 = step(orc, S2, row(pert, 0), dims)
        changed = [i for i in range(vh) if not bits_equal(o2[0, i], o_base[0, i])]
        assert changed == list(range(rep * j, rep * j + rep)), (j, changed)


def pin_unit_offsets(orc):
    """The same inputs placed in unit 0 and in the last unit give identical
    bits (the cross-layer slice of "Kestrel_VLLM #24", section 7)."""
    dims = (6, 2, 8, 8)
    N = 5
    r = _rng(17)
    S, inp = rand_inputs(r, N, dims)
    for name, a in inp.items():
        a[:, N - 1] = a[:, 0]
    S[N - 1] = S[0]
    o = step(orc, S, row(inp, 0), dims)
    assert bits_equal(S[0], S[N - 1]) and bits_equal(o[0], o[N - 1])
    assert not bits_equal(o[0], o[1])


def pin_step_m_equals_steps(orc):
    """M sequential rows in one call == M single steps (bit for bit)."""
    dims = (6, 2, 8, 4)
    M = 4
    r = _rng(19)
    S, inp = rand_inputs(r, 3, dims, M=M)
    S1 = S.copy()
    o_m = np.zeros((M,) + (3, dims[0], dims[3]), np.float32)
    orc.gdn_step_m(S, *(inp[n] for n in ("q", "k", "v", "g", "beta")), o_m, M, dims)
    for m in range(M):
        o1 = step(orc, S1, row(inp, m), dims)
        assert bits_equal(o1, o_m[m]), m
    assert bits_equal(S, S1)
    assert not bits_equal(o_m[0], o_m[1])


def pin_mark_rollback(orc):
    """mark -> step_m -> rollback(a) equals a single steps from the mark (bit
    for bit); rollback(0) restores the marked bytes; the snapshot is one-shot;
    the check discriminates (without the restore, the states differ)."""
    dims = (6, 2, 8, 4)
    vh, kh, kd, vd = dims
    M, N = 5, 4
    conv_dim, ck = 12, 4
    r = _rng(23)
    S, inp = rand_inputs(r, N, dims, M=M)
    hist = r.normal(size=(N, ck - 1, conv_dim)).astype(np.float32)
    xc = r.normal(size=(M, N, conv_dim)).astype(np.float32)
    S_mark, hist_mark = S.copy(), hist.copy()
    slab = orc.slab(N, dims, hist_floats=(ck - 1) * conv_dim)
    slab.mark(S, hist)
    assert slab.armed
    o_m = np.zeros((M, N, vh, vd), np.float32)
    orc.gdn_step_m(S, *(inp[n] for n in ("q", "k", "v", "g", "beta")), o_m, M, dims)
    for u in range(N):
        orc.conv_push(hist[u], xc[0, u].copy(), conv_dim, ck)
    assert not bits_equal(S, S_mark)
    acc = np.array([0, 1, 3, M], np.int32)
    slab.rollback(S, hist, inp, M, acc, xc_raw=xc, conv_dim=conv_dim, ck=ck)
    assert not slab.armed
    # expected: a single steps per unit from the marked state
    for u in range(N):
        Su = S_mark[u:u + 1].copy()
        hu = hist_mark[u].copy()
        for m in range(acc[u]):
            x = {n: np.ascontiguousarray(a[m, u:u + 1]) for n, a in inp.items()}
            step(orc, Su, x, dims)
            orc.conv_push(hu, xc[m, u].copy(), conv_dim, ck)
        assert bits_equal(S[u:u + 1], Su), u
        assert bits_equal(hist[u], hu), u
        if acc[u] == 0:
            assert bits_equal(S[u], S_mark[u]) and bits_equal(hist[u], hist_mark[u])
    # one-shot: a second rollback is refused and changes nothing
    S_before = S.copy()
    with pytest.raises(ValueError):
        slab.rollback(S, hist, inp, M, acc, xc_raw=xc, conv_dim=conv_dim, ck=ck)
    assert bits_equal(S, S_before)
    # out-of-range accepted is refused
    slab.mark(S, hist)
    with pytest.raises(ValueError):
        slab.rollback(S, hist, inp, M, np.array([0, 1, M + 1, 0], np.int32),
                      xc_raw=xc, conv_dim=conv_dim, ck=ck)


def pin_history_is_last_raw_frames(orc):
    """After T >= ck-1 pushes the history holds the last ck-1 raw inputs,
    oldest first, bit for bit; after fewer pushes it keeps the newest old
    frames in front of them."""
    conv_dim, ck = 10, 4
    r = _rng(29)
    h0 = r.normal(size=(ck - 1, conv_dim)).astype(np.float32)
    raws = r.normal(size=(6, conv_dim)).astype(np.float32)
    for T in range(7):
        h = h0.copy()
        for t in range(T):
            orc.conv_push(h, raws[t].copy(), conv_dim, ck)
        seq = np.concatenate([h0, raws[:T]], axis=0)
        assert bits_equal(h, seq[-(ck - 1):]), T


# --------------------------------------------------------------------------
# the front end
# --------------------------------------------------------------------------

FE_DIMS = (6, 2, 8, 8)       # vh, kh, kd, vd -> conv_dim = 80


def fe_case(r, B, dims=FE_DIMS, dim=64, ck=4, zero_params=True):
    vh, kh, kd, vd = dims
    cd = 2 * kh * kd + vh * vd
    d = dict(
        x=r.normal(size=(B, dim)).astype(np.float32),
        Wa=r.normal(0, 0.1, (vh, dim)).astype(np.float32),
        Wb=r.normal(0, 0.1, (vh, dim)).astype(np.float32),
        A_log=(np.zeros(vh) if zero_params else r.normal(0, 0.5, vh)).astype(np.float32),
        dt_bias=(np.zeros(vh) if zero_params else r.normal(0, 0.5, vh)).astype(np.float32),
        xc_raw=r.normal(size=(B, cd)).astype(np.float32),
        hist=r.normal(size=(B, ck - 1, cd)).astype(np.float32),
        conv_w=r.normal(0, 0.5, (cd, ck)).astype(np.float32),
    )
    return d


def run_fe(orc, d, dims=FE_DIMS, ck=4):
    vh, kh, kd, vd = dims
    B = d["x"].shape[0]
    out = dict(q=np.zeros((B, kh, kd), np.float32), k=np.zeros((B, kh, kd), np.float32),
               v=np.zeros((B, vh, vd), np.float32), g=np.zeros((B, vh), np.float32),
               beta=np.zeros((B, vh), np.float32))
    orc.gdn_frontend(d["x"], d["Wa"], d["Wb"], d["A_log"], d["dt_bias"], d["xc_raw"],
                     d["hist"], d["conv_w"], out["q"], out["k"], out["v"], out["g"],
                     out["beta"], dims, ck)
    return out


def pin_fe_gemv_gate_beta(orc):
    """A_log = dt_bias = 0: beta = sigmoid(Wb x) and g = -softplus(Wa x),
    against a double-precision matrix product and library sigmoid/softplus;
    beta comes from Wb, the gate from Wa."""
    r = _rng(31)
    d = fe_case(r, 3)
    out = run_fe(orc, d)
    a = d["x"].astype(np.float64) @ d["Wa"].astype(np.float64).T
    b = d["x"].astype(np.float64) @ d["Wb"].astype(np.float64).T
    assert_close(out["beta"], expit(b), "beta")
    assert_close(out["g"], -np.logaddexp(0.0, a), "g")


def pin_fe_gate_closed_forms(orc):
    """x = 0: beta = 1/2 exactly and g = -exp(A_log) softplus(dt_bias);
    at A_log = dt_bias = 0, g = -ln 2.  Sign symmetry: beta(x) + beta(-x) = 1,
    g(-x) - g(x) = a = Wa x (softplus(a) - softplus(-a) = a).  The guarded
    branches at |xa| > 20 agree with softplus."""
    r = _rng(37)
    d = fe_case(r, 2)
    d["x"][:] = 0.0
    out = run_fe(orc, d)
    assert np.all(out["beta"] == 0.5)
    assert np.allclose(out["g"], -np.log(2.0), rtol=2e-7, atol=0)
    d = fe_case(r, 2)
    p = run_fe(orc, d)
    d["x"] = -d["x"]
    n = run_fe(orc, d)
    assert_close(p["beta"].astype(np.float64) + n["beta"], np.ones_like(p["beta"]), "sym beta",
                 rel=3e-7, floor=0)
    a = -d["x"].astype(np.float64) @ d["Wa"].astype(np.float64).T
    assert_close(n["g"].astype(np.float64) - p["g"], a, "sym g", rel=1e-5, floor=1e-6)
    for xa in (-30.0, -20.5, -19.5, 0.3, 19.5, 20.5, 30.0):
        d = fe_case(r, 1, zero_params=False)
        d["x"][:] = 0.0
        d["dt_bias"][:] = xa
        out = run_fe(orc, d)
        want = -np.exp(d["A_log"].astype(np.float64)) * np.logaddexp(0.0, np.float64(np.float32(xa)))
        assert_close(out["g"][0], want, f"softplus branch {xa}", rel=1e-6, floor=1e-30)


def _silu(x):
    x = x.astype(np.float64)
    return x * expit(x)


def _normed(c, kh, kd, scale):
    c = c.reshape(kh, kd)
    return c / np.sqrt(np.sum(c * c, axis=1, keepdims=True) + 1e-6) * scale


def pin_fe_conv_taps_split_norm(orc):
    """A one-hot conv weight on the last tap gives silu(raw); on tap j < ck-1
    it gives silu(history frame j).  The conv output splits at 0, kh*kd,
    2*kh*kd into q | k | v; q and k heads are L2-normalised (q also scaled by
    1/sqrt(kd)), v is not normalised."""
    vh, kh, kd, vd = FE_DIMS
    w = kh * kd
    r = _rng(41)
    for tap in range(4):
        d = fe_case(r, 2)
        h0 = d["hist"].copy()
        d["conv_w"][:] = 0.0
        d["conv_w"][:, tap] = 1.0
        out = run_fe(orc, d)
        for b in range(2):
            src = d["xc_raw"][b] if tap == 3 else h0[b, tap]
            c = _silu(src)
            assert_close(out["v"][b].ravel(), c[2 * w:], f"v tap {tap}", rel=1e-6, floor=1e-7)
            assert_close(out["q"][b], _normed(c[:w], kh, kd, 1 / np.sqrt(kd)), "q", rel=1e-6, floor=1e-7)
            assert_close(out["k"][b], _normed(c[w:2 * w], kh, kd, 1.0), "k", rel=1e-6, floor=1e-7)


def pin_fe_norms(orc):
    """Per key head: sum k^2 = 1 and sum q^2 = 1/kd; an all-zero head stays
    zero (the epsilon sits inside the square root)."""
    vh, kh, kd, vd = FE_DIMS
    r = _rng(43)
    d = fe_case(r, 3)
    d["conv_w"][:kd, :] = 0.0           # q head 0 of every row: conv output 0
    out = run_fe(orc, d)
    sq = np.sum(out["q"].astype(np.float64) ** 2, axis=-1)
    sk = np.sum(out["k"].astype(np.float64) ** 2, axis=-1)
    assert np.all(out["q"][:, 0] == 0.0)
    assert np.allclose(sq[:, 1:], 1.0 / kd, rtol=1e-5, atol=0)
    assert np.allclose(sk, 1.0, rtol=1e-5, atol=0)


def pin_fe_history_advance(orc):
    """Each front-end call pushes its raw conv input into the history."""
    r = _rng(47)
    d = fe_case(r, 2)
    h0 = d["hist"].copy()
    raws = []
    for t in range(4):
        d["xc_raw"] = r.normal(size=d["xc_raw"].shape).astype(np.float32)
        raws.append(d["xc_raw"].copy())
        run_fe(orc, d)
        seq = np.concatenate([h0, np.stack(raws, axis=1)], axis=1)
        assert bits_equal(d["hist"], np.ascontiguousarray(seq[:, -3:])), t


# --------------------------------------------------------------------------
# gated RMSNorm of the output
# --------------------------------------------------------------------------

def _gnorm(orc, o, z, w, eps):
    out = np.zeros_like(o)
    orc.gated_norm(o, z, w, eps, out)
    return out


def pin_gated_norm_closed_forms(orc):
    """out = (o / sqrt(mean(o^2) + eps)) * w * silu(z), per row:
    z = 0 gives 0 exactly; z = 30 gives silu = 30 exactly in fp32, so with
    w = 1 and eps = 0 the mean square of out is 900 (a mean over vd, not a
    sum); scaling o by 4 leaves out unchanged bit for bit (eps = 0); a row of
    equal entries c = 1e-3 with eps = 1e-6 gives 30/sqrt(2) (eps inside the
    root); the gate enters as z * sigmoid(z); w scales each column."""
    r = _rng(59)
    vd = 16
    o = r.normal(size=(3, vd)).astype(np.float32)
    w1 = np.ones(vd, np.float32)
    assert np.all(_gnorm(orc, o, np.zeros_like(o), w1, 1e-6) == 0.0)
    z30 = np.full_like(o, 30.0)
    out = _gnorm(orc, o, z30, w1, 0.0)
    assert np.allclose(np.mean(out.astype(np.float64) ** 2, axis=1), 900.0, rtol=2e-6)
    assert bits_equal(_gnorm(orc, (o * 4).astype(np.float32), z30, w1, 0.0), out)
    c = np.full((1, vd), 1e-3, np.float32)
    assert np.allclose(_gnorm(orc, c, np.full_like(c, 30.0), w1, 1e-6), 30 / np.sqrt(2), rtol=1e-5)
    z = r.normal(size=o.shape).astype(np.float32)
    base = _gnorm(orc, o, z30, w1, 1e-6) / 30.0
    assert_close(_gnorm(orc, o, z, w1, 1e-6), base * z * expit(z.astype(np.float64)),
                 "silu gate", rel=1e-5, floor=1e-7)
    w = r.normal(size=vd).astype(np.float32)
    assert_close(_gnorm(orc, o, z30, w, 1e-6), (base * 30.0) * w, "weight", rel=1e-6, floor=1e-7)


# --------------------------------------------------------------------------
# dense projections (in_proj / out_proj)
# --------------------------------------------------------------------------

def _proj(orc, x, W):
    y = np.zeros((x.shape[0], W.shape[0]), np.float32)
    orc.proj(np.ascontiguousarray(x), np.ascontiguousarray(W), y)
    return y


def pin_proj_one_hot_and_exact(orc):
    """y = x W^T.  A one-hot row x = e_c selects column c of W exactly (each
    row with its own c, the last column included); small integer operands make
    every product and partial sum exact in fp32, so y equals the integer
    product; R != C so that a transposed operand cannot pass."""
    r = _rng(61)
    R, C = 7, 12
    W = r.normal(size=(R, C)).astype(np.float32)
    cols = [C - 1, 0, 5, 11, 3]
    x = np.zeros((len(cols), C), np.float32)
    for i, c in enumerate(cols):
        x[i, c] = 1.0
    y = _proj(orc, x, W)
    for i, c in enumerate(cols):
        assert bits_equal(y[i], np.ascontiguousarray(W[:, c])), (i, c)
    Wi = r.integers(-8, 9, size=(R, C))
    xi = r.integers(-8, 9, size=(4, C))
    y = _proj(orc, xi.astype(np.float32), Wi.astype(np.float32))
    assert np.array_equal(y.astype(np.int64), xi @ Wi.T)


def pin_proj_left_fold_in_fp32(orc):
    """The sum over c is a left fold with every partial sum rounded to fp32:
    for the terms (2^24, 1, -2^24, 1) the fold gives ((2^24 + 1) - 2^24) + 1
    = 0 + 1 = 1 (2^24 + 1 rounds to 2^24), while the exact sum, and a fold in
    the reverse order, give 2."""
    W = np.array([[2.0 ** 24, 1.0, -(2.0 ** 24), 1.0]], np.float32)
    x = np.ones((1, 4), np.float32)
    assert _proj(orc, x, W)[0, 0] == 1.0


def pin_proj_brute_force_fp64(orc):
    """Random operands at the layer's inner size: within 1e-6 of the sum of
    |W x| terms from a double-precision dot product (a dropped or misplaced
    term is about 2e-4 of that sum); M rows in one call equal one-row calls."""
    r = _rng(67)
    R, C = 24, 5120
    W = r.normal(0, 0.02, size=(R, C)).astype(np.float32)
    x = r.normal(size=(3, C)).astype(np.float32)
    y = _proj(orc, x, W)
    W64, x64 = W.astype(np.float64), x.astype(np.float64)
    ref = x64 @ W64.T
    mag = np.abs(x64) @ np.abs(W64).T
    assert np.all(np.abs(y - ref) <= 1e-6 * mag)
    for i in range(3):
        assert bits_equal(_proj(orc, x[i:i + 1], W)[0], y[i])


def pin_half_to_float_all_patterns(orc):
    """binary16 -> binary32 for all 65536 bit patterns equals numpy's
    float16 conversion (NaN for NaN): zeros, subnormals, normals, infinities,
    both signs."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.half_to_float(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert bits_equal(got[~nan], ref[~nan])


def _q4_case(r, R, C):
    q = r.integers(0, 256, size=(R, C // 2)).astype(np.uint8)
    sc = (r.normal(0, 0.01, size=(R, C // 32)) + 0.0).astype(np.float16)
    return q, np.ascontiguousarray(sc.view(np.uint16))


def _q4_decode(q, scale):
    """numpy decode: low nibble is the even element, two's complement, times
    the block's scale (float16 -> float32 is exact, so is the product)."""
    R = q.shape[0]
    nib = np.stack([q & 0x0F, q >> 4], axis=-1).reshape(R, -1).astype(np.int32)
    n = ((nib ^ 8) - 8).astype(np.float32)
    s = scale.view(np.float16).astype(np.float32)
    return np.ascontiguousarray(n * np.repeat(s, 32, axis=1))


def pin_proj_q4_is_the_decoded_f32_projection(orc):
    """The 4-bit projection equals the f32 projection of the weights decoded
    by numpy (nibble order, sign, 32-weight scale blocks, the scale's
    conversion), bit for bit; a one-hot row returns the decoded column."""
    r = _rng(73)
    R, C = 24, 256
    q, sc = _q4_case(r, R, C)
    x = r.normal(size=(3, C)).astype(np.float32)
    y4 = np.zeros((3, R), np.float32)
    orc.proj_q4(x, q, sc, y4)
    Wd = _q4_decode(q, sc)
    assert bits_equal(y4, _proj(orc, x, Wd))
    e = np.zeros((1, C), np.float32)
    e[0, C - 33] = 1.0
    y1 = np.zeros((1, R), np.float32)
    orc.proj_q4(e, q, sc, y1)
    assert bits_equal(y1[0], np.ascontiguousarray(Wd[:, C - 33]))


def pin_proj_q4_closed_form(orc):
    """Byte 0x9F holds -1 (low nibble 0xF) then -7 (high nibble 0x9); with
    scale 0.5 and x = (1, 10) the output is -0.5 - 35 = -35.5; 0x80 is 0 then
    -8 (the most negative value)."""
    C = 32
    q = np.zeros((2, C // 2), np.uint8)
    q[0, 0] = 0x9F
    q[1, 0] = 0x80
    sc = np.array([[0.5], [0.25]], np.float16).view(np.uint16)
    x = np.zeros((1, C), np.float32)
    x[0, 0], x[0, 1] = 1.0, 10.0
    y = np.zeros((1, 2), np.float32)
    orc.proj_q4(x, q, np.ascontiguousarray(sc), y)
    assert y[0, 0] == -35.5 and y[0, 1] == -20.0


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


def test_oracle_refuses_bad_arguments(orc):
    dims = (5, 2, 4, 4)                      # vh not a multiple of kh
    S = np.zeros((1, 5, 4, 4), np.float32)
    z = np.zeros(64, np.float32)
    with pytest.raises(ValueError):
        orc.gdn_step(S, z, z, z, z, z, z, dims)


def test_frontend_m_rows_equal_single_calls(orc):
    """The oracle's M-row front end is M single-row calls with the history
    advancing once per row (row strides of x, xc_raw and every output)."""
    vh, kh, kd, vd = FE_DIMS
    r = _rng(53)
    M, B = 3, 2
    d = fe_case(r, B)
    xs = r.normal(size=(M, B, d["x"].shape[1])).astype(np.float32)
    raws = r.normal(size=(M, B, d["xc_raw"].shape[1])).astype(np.float32)
    h_m = d["hist"].copy()
    outs = dict(q=np.zeros((M, B, kh, kd), np.float32), k=np.zeros((M, B, kh, kd), np.float32),
                v=np.zeros((M, B, vh, vd), np.float32), g=np.zeros((M, B, vh), np.float32),
                beta=np.zeros((M, B, vh), np.float32))
    orc.gdn_frontend_m(xs, d["Wa"], d["Wb"], d["A_log"], d["dt_bias"], raws, h_m, d["conv_w"],
                       outs["q"], outs["k"], outs["v"], outs["g"], outs["beta"], FE_DIMS)
    for m in range(M):
        d["x"] = np.ascontiguousarray(xs[m])
        d["xc_raw"] = np.ascontiguousarray(raws[m])
        one = run_fe(orc, d)
        for n in ("q", "k", "v", "g", "beta"):
            assert bits_equal(outs[n][m], one[n]), (n, m)
    assert bits_equal(h_m, d["hist"])
