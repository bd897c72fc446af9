"""GPU parity: the gfx950 kernels (through the C ABI) against the CPU oracle.

Floating point: per element |x - r| <= max(1e-5 |r|, 1e-6) on o, S and the
front-end outputs.  Bit-exact: step_m against M single steps, rollback against
single steps from the mark, rollback(0) against the marked bytes, the reset
gate's closed form, the conv history, repeated runs.  The full-size
workloads are checked on every unit in test_gpu_full_size.py.
"""
import ctypes as C

import numpy as np
import pytest
import torch

import gated_deltanet_recurrent_amd as gdn
import synth
from tests.helpers import assert_close, bits_equal, max_rel_pages

pytestmark = pytest.mark.gpu

NAMES = ("q", "k", "v", "g", "beta")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    gdn.lib()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def say(*a):
    print(*a, flush=True)


def host(t):
    return np.ascontiguousarray(t.detach().cpu().numpy())


def host_rows(inp, idx):
    """Inputs [M][N][...] restricted to units idx, on the host."""
    ii = torch.as_tensor(idx, device=inp["q"].device)
    return {n: np.ascontiguousarray(host(inp[n].index_select(1, ii))) for n in NAMES}


def row0(inp):
    return {n: inp[n][0] for n in NAMES}


def ref_steps(orc, S, inp, dims, rows):
    """Oracle: `rows` chained single steps; returns list of o."""
    outs = []
    for m in range(rows):
        x = {n: np.ascontiguousarray(inp[n][m]) for n in NAMES}
        o = np.zeros((S.shape[0], dims[0], dims[3]), np.float32)
        orc.gdn_step(S, x["q"], x["k"], x["v"], x["g"], x["beta"], o, dims)
        outs.append(o)
    return outs


def ref_cycle(orc, S0, inp, dims, acc, hist0=None, xc=None):
    """Oracle of one speculative cycle on host copies: mark(S, hist), M
    steps (o for every row), rollback(accepted) replaying the history frames.
    Returns (o [M][N][vh][vd], S after the M steps, S after the rollback,
    history after the rollback or None)."""
    vh, kh, kd, vd = dims
    M, N = inp["q"].shape[:2]
    S = np.ascontiguousarray(S0).copy()
    h = None if hist0 is None else np.ascontiguousarray(hist0).copy()
    cd = 0 if xc is None else xc.shape[-1]
    rs = orc.slab(N, dims, hist_floats=3 * cd)
    rs.mark(S, h)
    o = np.zeros((M, N, vh, vd), np.float32)
    orc.gdn_step_m(S, *(inp[n] for n in NAMES), o, M, dims)
    S_m = S.copy()
    rs.rollback(S, h, inp, M, np.asarray(acc, np.int32), xc_raw=xc, conv_dim=cd, ck=4)
    return o, S_m, S, h


def ref_gated(orc, o_ref, z, w, eps):
    """The oracle's gated RMSNorm of o_ref and the gated output's per-element
    absolute floor: o's floor (1e-6) carried through the per-head scale
    s = w silu(z) / sqrt(mean(o^2) + eps)."""
    out = np.zeros_like(o_ref)
    orc.gated_norm(o_ref, z, w, eps, out)
    o64, z64 = o_ref.astype(np.float64), z.astype(np.float64)
    rinv = 1.0 / np.sqrt(np.mean(o64 ** 2, axis=-1, keepdims=True) + eps)
    scale = np.abs(rinv * w.astype(np.float64) * z64 / (1.0 + np.exp(-z64)))
    return out, 1e-6 * scale


# ---------------------------------------------------------------------------
# single steps, small sizes: every element of every step
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dims,N,T", [
    (synth.DIMS128, 1, 64),          # single sequence, one layer, 64 decode steps
    (synth.DIMS128, 7, 4),
    (synth.DIMS64, 5, 6),
    ((6, 2, 128, 128), 3, 5),
    ((4, 4, 64, 64), 2, 5),
    ((8, 1, 128, 128), 2, 3),
    ((6, 2, 64, 64), 3, 4),          # kd = 64, vh not a multiple of 4: one tile per workgroup
    ((1, 1, 128, 128), 4, 3),        # one head
    ((1, 1, 64, 64), 5, 3),
])
def test_step_chain_parity(orc, dims, N, T):
    say(f"step chain dims={dims} N={N} T={T}")
    gen = synth.make_gen(0, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=T, device="cuda")
    S_ref = host(S)
    inp_h = {n: host(inp[n]) for n in NAMES}
    S_h = S_ref.copy()
    worst = 0.0
    for m in range(T):
        o = gdn.step(S, *(inp[n][m] for n in NAMES))
        x = {n: inp_h[n][m:m + 1] for n in NAMES}
        o_ref = ref_steps(orc, S_h, x, dims, 1)[0]
        assert_close(host(o), o_ref, f"o step {m}")
        assert_close(host(S), S_h, f"S step {m}")
        worst = max(worst, max_rel_pages(host(o), o_ref))
    say(f"  worst max|err|/max|ref| over steps = {worst:.3e}")


def test_step_writes_every_output_and_is_deterministic():
    dims = synth.DIMS128
    N = 9
    gen = synth.make_gen(1, "cuda")
    S0 = synth.state(gen, N, dims, device="cuda")
    inp = row0(synth.step_inputs(gen, N, dims, device="cuda"))
    runs = []
    for _ in range(2):
        S = S0.clone()
        o = torch.full((N, dims[0], dims[3]), float("nan"), device="cuda")
        gdn.step(S, *(inp[n] for n in NAMES), o=o)
        assert not torch.isnan(o).any()
        runs.append((host(S), host(o)))
    assert bits_equal(runs[0][0], runs[1][0]) and bits_equal(runs[0][1], runs[1][1])


def test_reset_gate_bit_exact_vs_oracle(orc):
    """g = -inf: S' = fl(k fl(v beta)) on both sides, bit for bit."""
    for dims in (synth.DIMS128, synth.DIMS64):
        N = 3
        gen = synth.make_gen(2, "cuda")
        S = synth.state(gen, N, dims, device="cuda")
        inp = row0(synth.step_inputs(gen, N, dims, device="cuda"))
        inp["g"].fill_(float("-inf"))
        S_h = host(S)
        x = {n: host(inp[n]) for n in NAMES}
        o = gdn.step(S, *(inp[n] for n in NAMES))
        o_ref = np.zeros((N, dims[0], dims[3]), np.float32)
        orc.gdn_step(S_h, x["q"], x["k"], x["v"], x["g"], x["beta"], o_ref, dims)
        assert bits_equal(host(S), S_h)
        # and the read-out: o = tmp (k . q) with tmp = v beta, per value head
        assert_close(host(o), o_ref, "o reset gate")
        rep = dims[0] // dims[1]
        kq = np.einsum("nhd,nhd->nh", x["k"].astype(np.float64), x["q"].astype(np.float64))
        o_closed = (x["v"].astype(np.float64) * x["beta"].astype(np.float64)[..., None]
                    * np.repeat(kq, rep, axis=1)[..., None])
        assert_close(host(o), o_closed, "o reset gate closed form")


@pytest.mark.parametrize("dims,N,M", [(synth.DIMS128, 3, 1), (synth.DIMS64, 3, 1),
                                      (synth.DIMS128, 3, 3), (synth.DIMS128, 24, 3)])
def test_nan_stays_in_its_tile(orc, dims, N, M):
    """A NaN planted in one state element spreads only as IEEE arithmetic
    carries it inside its own (unit, head) tile: after M steps (single-step,
    few-tile and many-tile M-step kernels) the NaN positions of S and o equal
    the oracle's, the finite elements agree within tolerance, and every other
    tile stays finite (a wrong tile, row or column offset would spread it)."""
    say(f"nan isolation dims={dims} N={N} M={M}")
    vh, kh, kd, vd = dims
    gen = synth.make_gen(17, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    u, h, i, j = 1, vh // 2 + 1, kd // 3, vd - 2
    S[u, h, i, j] = float("nan")
    S_h = host(S)
    x = {n: host(inp[n]) for n in NAMES}
    if M == 1:
        o = gdn.step(S, *(inp[n][0] for n in NAMES)).unsqueeze(0)
    else:
        o = gdn.step_m(S, *(inp[n] for n in NAMES))
    o_ref = np.stack(ref_steps(orc, S_h, x, dims, M))
    got_S, got_o = host(S), host(o)
    for got, ref, what in ((got_S, S_h, "S"), (got_o, o_ref, "o")):
        nan = np.isnan(ref)
        assert nan.any(), what
        assert np.array_equal(np.isnan(got), nan), what
        assert_close(got[~nan], ref[~nan], what)
    others = np.ones((N, vh), bool)
    others[u, h] = False
    assert np.isfinite(got_S[others]).all() and np.isfinite(got_o[:, others]).all()


def test_unit_offsets_identical():
    dims = synth.DIMS128
    N = 6
    gen = synth.make_gen(3, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = row0(synth.step_inputs(gen, N, dims, device="cuda"))
    S[N - 1] = S[0]
    for n in NAMES:
        inp[n][N - 1] = inp[n][0]
    o = gdn.step(S, *(inp[n] for n in NAMES))
    assert bits_equal(host(S[0]), host(S[N - 1])) and bits_equal(host(o[0]), host(o[N - 1]))


def test_step_on_side_stream(orc):
    dims = synth.DIMS64
    N = 4
    gen = synth.make_gen(4, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = row0(synth.step_inputs(gen, N, dims, device="cuda"))
    S_h = host(S)
    x = {n: host(inp[n]) for n in NAMES}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o = gdn.step(S, *(inp[n] for n in NAMES))
    torch.cuda.current_stream().wait_stream(side)
    o_ref = np.zeros((N, dims[0], dims[3]), np.float32)
    orc.gdn_step(S_h, x["q"], x["k"], x["v"], x["g"], x["beta"], o_ref, dims)
    assert_close(host(o), o_ref, "o side stream")
    assert_close(host(S), S_h, "S side stream")


# ---------------------------------------------------------------------------
# M-step, mark / rollback
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dims,M", [(synth.DIMS128, 8), (synth.DIMS64, 5), (synth.DIMS128, 1),
                                    (synth.DIMS128, 64), ((6, 2, 64, 64), 4),
                                    ((1, 1, 128, 128), 8), ((6, 2, 64, 64), 12)])
def test_step_m_bit_exact_and_parity(orc, dims, M):
    say(f"step_m dims={dims} M={M}")
    N = 3
    gen = synth.make_gen(5, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    S1 = S.clone()
    S_h = host(S)
    o_m = gdn.step_m(S, *(inp[n] for n in NAMES))
    for m in range(M):
        o1 = gdn.step(S1, *(inp[n][m] for n in NAMES))
        assert bits_equal(host(o1), host(o_m[m])), m
    assert bits_equal(host(S), host(S1))
    o_ref = np.zeros((M, N, dims[0], dims[3]), np.float32)
    orc.gdn_step_m(S_h, *(host(inp[n]) for n in NAMES), o_ref, M, dims)
    assert_close(host(o_m), o_ref, "o step_m")
    assert_close(host(S), S_h, "S step_m")


def test_single_step_geometries_agree_at_the_tile_boundary():
    """Single steps of fewer than 1024 tiles run the split geometry (ungated),
    larger ones the wide geometry: 22 units (1056 tiles) against their first
    21 units (1008 tiles) and a single unit, bit for bit, ungated and gated."""
    say("single-step geometries at 1024 tiles")
    dims = synth.DIMS128
    vh, vd = dims[0], dims[3]
    N = 22
    gen = synth.make_gen(61, "cuda")
    S0 = synth.state(gen, N, dims, device="cuda")
    inp = row0(synth.step_inputs(gen, N, dims, device="cuda"))
    z = torch.randn((1, N, vh, vd), generator=gen, device="cuda")
    w = 1.0 + 0.1 * torch.randn((vd,), generator=gen, device="cuda")

    def run(n):
        S = S0[:n].clone()
        o = host(gdn.step(S, *(inp[k][:n].contiguous() for k in NAMES)))
        Sg = S0[:n].clone()
        og = host(gdn.step_gated(Sg, *(inp[k][:n].contiguous().unsqueeze(0) for k in NAMES),
                                 z[:, :n].contiguous(), w, 1e-6))
        return o, host(S), og, host(Sg)

    full = run(N)
    for n in (N - 1, 1):
        part = run(n)
        for a, b in zip(full, part):
            sl = np.ascontiguousarray(a[:, :n] if a.ndim == 4 and a.shape[0] == 1 else a[:n])
            assert bits_equal(sl, b), n


@pytest.mark.parametrize("dims,N", [(synth.DIMS128, 24), (synth.DIMS64, 11), (synth.DIMS128, 8)])
@pytest.mark.parametrize("M", [2, 8])
def test_m_step_geometries_agree(orc, dims, N, M):
    """Launches of fewer than 1024 tiles, M <= 8 and tiles x M <= 2048 run the
    few-tile kernels (split when ungated at kd = 128, else the wide geometry
    step after step), the others the deep geometry: a launch over N units
    against launches over slices of 1 and 3 units, bit for bit, for step_m,
    the gated step, verify_m_gated (no state store) and commit with per-unit
    counts (including 0 and M).  N = 24 and 11 are deep at both M; N = 8 (384
    tiles) is deep at M = 8 and few-tile at M = 2."""
    say(f"M-step geometries dims={dims} N={N} M={M}")
    vh, vd = dims[0], dims[3]
    gen = synth.make_gen(41 + M, "cuda")
    S0 = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    z = torch.randn((M, N, vh, vd), generator=gen, device="cuda")
    w = 1.0 + 0.1 * torch.randn((vd,), generator=gen, device="cuda")
    acc = torch.tensor([(3 * u) % (M + 1) for u in range(N)], dtype=torch.int32, device="cuda")

    def run(lo, hi):
        sl = {n: inp[n][:, lo:hi].contiguous() for n in NAMES}
        zz = z[:, lo:hi].contiguous()
        S = S0[lo:hi].clone()
        o = host(gdn.step_m(S, *(sl[n] for n in NAMES)))
        Sg = S0[lo:hi].clone()
        og = host(gdn.step_gated(Sg, *(sl[n] for n in NAMES), zz, w, 1e-6))
        Sv = S0[lo:hi].clone()
        ov = host(gdn.verify_m_gated(Sv, *(sl[n] for n in NAMES), zz, w, 1e-6))
        gdn.commit(Sv, acc[lo:hi].contiguous(), *(sl[n] for n in NAMES))
        return o, host(S), og, host(Sg), ov, host(Sv)

    full = run(0, N)
    for lo, hi in ((0, 1), (N - 3, N), (N // 2, N // 2 + 1)):
        part = run(lo, hi)
        for i, (a, b) in enumerate(zip(full, part)):
            sl = (slice(None), slice(lo, hi)) if a.ndim == 4 and i % 2 == 0 else slice(lo, hi)
            assert bits_equal(np.ascontiguousarray(a[sl]), b), (lo, hi, i)
    # the full launch against the oracle: step_m, gated outputs, and the
    # verify + commit cycle's state (= mark, M steps, rollback to the counts)
    o, S, og, Sg, ov, Sv = full
    x_h = {n: host(inp[n]) for n in NAMES}
    o_ref, S_m, S_rb, _ = ref_cycle(orc, host(S0), x_h, dims, host(acc))
    assert_close(o, o_ref, "o step_m")
    assert_close(S, S_m, "S step_m")
    assert bits_equal(Sg, S)
    g_ref, g_floor = ref_gated(orc, o_ref, host(z), host(w), 1e-6)
    assert_close(og, g_ref, "gated out", floor=g_floor)
    assert_close(ov, g_ref, "verify_m_gated out", floor=g_floor)
    assert_close(Sv, S_rb, "S after commit")


@pytest.mark.parametrize("dims", [synth.DIMS128, synth.DIMS64])
def test_mark_rollback_bit_exact(orc, dims):
    """mark -> step_m(M) -> rollback(accepted): each unit equals accepted[u]
    GPU single steps from the mark (S and history, bit for bit); 0 restores
    the marked bytes; M reproduces step_m; a second rollback is refused."""
    say(f"mark/rollback dims={dims}")
    vh, kh, kd, vd = dims
    N, M = 6, 5
    cd = synth.conv_dim_of(dims)
    gen = synth.make_gen(6, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    hist = torch.randn((N, 3, cd), generator=gen, device="cuda")
    xc = torch.randn((M, N, cd), generator=gen, device="cuda")
    S_mark, hist_mark = S.clone(), hist.clone()
    slab = gdn.Slab(N, dims, hist_floats_per_unit=3 * cd)
    slab.mark(S, hist)
    assert slab.armed == 3
    gdn.step_m(S, *(inp[n] for n in NAMES))
    S_after_m = S.clone()
    assert not bits_equal(host(S), host(S_mark))
    hist.add_(1.0)                                 # the history advanced meanwhile
    acc = [0, 1, 2, M, 3, M - 1]
    slab.rollback(S, acc, *(inp[n] for n in NAMES), hist=hist, xc_raw=xc)
    assert slab.armed == 0
    # expected: GPU single steps from the mark
    S_exp = S_mark.clone()
    h_exp = host(hist_mark)
    xc_h = host(xc)
    for u in range(N):
        Su = S_exp[u:u + 1]
        for m in range(acc[u]):
            gdn.step(Su, *(inp[n][m, u:u + 1].contiguous() for n in NAMES))
        seq = np.concatenate([h_exp[u], xc_h[:acc[u], u]], axis=0)
        h_exp[u] = seq[-3:]
    assert bits_equal(host(S), host(S_exp))
    assert bits_equal(host(hist), h_exp)
    assert bits_equal(host(S[0]), host(S_mark[0]))
    assert bits_equal(host(S[3]), host(S_after_m[3]))
    # oracle agrees within tolerance
    S_ref = host(S_mark)
    rs = orc.slab(N, dims, hist_floats=3 * cd)
    h_ref = host(hist_mark)
    rs.mark(S_ref, h_ref)
    o_tmp = np.zeros((M, N, vh, vd), np.float32)
    orc.gdn_step_m(S_ref, *(host(inp[n]) for n in NAMES), o_tmp, M, dims)
    rs.rollback(S_ref, h_ref, {n: host(inp[n]) for n in NAMES}, M, np.array(acc, np.int32),
                xc_raw=xc_h, conv_dim=cd, ck=4)
    assert_close(host(S), S_ref, "S rollback vs oracle")
    assert bits_equal(host(hist), h_ref)
    # one-shot
    with pytest.raises(gdn.GdnError):
        slab.rollback(S, acc, *(inp[n] for n in NAMES), hist=hist, xc_raw=xc)


@pytest.mark.parametrize("dims,M", [(synth.DIMS128, 8), (synth.DIMS64, 12), (synth.DIMS128, 1)])
def test_mark_step_m_fused(orc, dims, M):
    """gdn_mark_step_m == gdn_mark + gdn_step_m: same state, outputs and
    snapshot bits (rollback(0) restores the marked bytes), history marked."""
    say(f"mark_step_m dims={dims} M={M}")
    vh, kh, kd, vd = dims
    N = 5
    cd = synth.conv_dim_of(dims)
    gen = synth.make_gen(13, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    hist = torch.randn((N, 3, cd), generator=gen, device="cuda")
    S_mark = S.clone()
    S2 = S.clone()
    slab = gdn.Slab(N, dims, hist_floats_per_unit=3 * cd)
    o = slab.mark_step_m(S, *(inp[n] for n in NAMES), hist=hist)
    assert slab.armed == 3
    slab2 = gdn.Slab(N, dims, hist_floats_per_unit=3 * cd)
    slab2.mark(S2, hist)
    o2 = gdn.step_m(S2, *(inp[n] for n in NAMES))
    assert bits_equal(host(S), host(S2)) and bits_equal(host(o), host(o2))
    o_ref, S_m, _, _ = ref_cycle(orc, host(S_mark), {n: host(inp[n]) for n in NAMES}, dims,
                                 [0] * N)
    assert_close(host(o), o_ref, "o mark_step_m")
    assert_close(host(S), S_m, "S mark_step_m")
    hist_mark = host(hist)
    hist.add_(1.0)
    slab.rollback(S, [0] * N, *(inp[n] for n in NAMES), hist=hist,
                  xc_raw=torch.zeros((M, N, cd), device="cuda"))
    assert bits_equal(host(S), host(S_mark))
    assert bits_equal(host(hist), hist_mark)
    # a mismatched slab is refused (by the binding's size check before the C
    # ABI's own GDN_ESTATE refusal, which the host-side tests exercise)
    small = gdn.Slab(N - 1, dims)
    with pytest.raises((gdn.GdnError, ValueError)):
        small.mark_step_m(S, *(inp[n] for n in NAMES))


@pytest.mark.parametrize("dims,B,M", [(synth.DIMS128, 4, 5), (synth.DIMS64, 3, 8),
                                      (synth.DIMS128, 2, 1)])
def test_mark_step_m_with_history_after_frontend_verify(orc, dims, B, M):
    """The fused mark's history protocol: frontend_verify_m (the history is
    only read), mark_step_m(S, hist), rollback(S, hist) to per-unit accepted
    lengths; outputs, state and history against the oracle's chain (mark,
    frontend_m, step_m, rollback), the history bit for bit."""
    say(f"mark_step_m with history dims={dims} B={B} M={M}")
    vh, kh, kd, vd = dims
    cd = synth.conv_dim_of(dims)
    gen = synth.make_gen(19, "cuda")
    S = synth.state(gen, B, dims, device="cuda")
    w = synth.frontend_weights(gen, dims, dim=1024, device="cuda")
    fe = synth.frontend_inputs(gen, B, dims, T=M, dim=1024, device="cuda")
    hist = fe["hist"]
    S_h, hist_h = host(S), host(hist)
    acc = [(2 * b + 1) % (M + 1) for b in range(B)]
    rows = gdn.frontend_verify_m(fe["x"], w["Wa"], w["Wb"], w["A_log"], w["dt_bias"],
                                 fe["xc_raw"], hist, w["conv_w"], dims)
    assert bits_equal(host(hist), hist_h)
    slab = gdn.Slab(B, dims, hist_floats_per_unit=3 * cd)
    o = slab.mark_step_m(S, *(rows[n] for n in NAMES), hist=hist)
    slab.rollback(S, acc, *(rows[n] for n in NAMES), hist=hist, xc_raw=fe["xc_raw"])
    wh = {n: host(t) for n, t in w.items()}
    ref = dict(q=np.zeros((M, B, kh, kd), np.float32), k=np.zeros((M, B, kh, kd), np.float32),
               v=np.zeros((M, B, vh, vd), np.float32), g=np.zeros((M, B, vh), np.float32),
               beta=np.zeros((M, B, vh), np.float32))
    h_fe = hist_h.copy()
    orc.gdn_frontend_m(host(fe["x"]), wh["Wa"], wh["Wb"], wh["A_log"], wh["dt_bias"],
                       host(fe["xc_raw"]), h_fe, wh["conv_w"], ref["q"], ref["k"], ref["v"],
                       ref["g"], ref["beta"], dims)
    for n in NAMES:
        assert_close(host(rows[n]), ref[n], f"frontend_verify_m {n}")
    o_ref, _, S_rb, h_rb = ref_cycle(orc, S_h, ref, dims, acc, hist_h, host(fe["xc_raw"]))
    assert_close(host(o), o_ref, "o")
    assert_close(host(S), S_rb, "S after rollback")
    assert bits_equal(host(hist), h_rb)


@pytest.mark.parametrize("dims,M", [(synth.DIMS64, 12), (synth.DIMS128, 10)])
def test_many_rows_prefetch_paths(orc, dims, M):
    """M > 8 rows run the prefetching instance: step_m, gated step and
    rollback against single steps (bits) and the oracle."""
    say(f"prefetch paths dims={dims} M={M}")
    vh, kh, kd, vd = dims
    N = 3
    gen = synth.make_gen(14, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    S0 = S.clone()
    S_h = host(S)
    slab = gdn.Slab(N, dims)
    slab.mark(S)
    o = gdn.step_m(S, *(inp[n] for n in NAMES))
    S1 = S0.clone()
    for m in range(M):
        o1 = gdn.step(S1, *(inp[n][m] for n in NAMES))
        assert bits_equal(host(o1), host(o[m])), m
    assert bits_equal(host(S), host(S1))
    o_ref = np.zeros((M, N, vh, vd), np.float32)
    orc.gdn_step_m(S_h, *(host(inp[n]) for n in NAMES), o_ref, M, dims)
    assert_close(host(o), o_ref, "o many rows")
    assert_close(host(S), S_h, "S many rows")
    acc = [M, 9, 2]
    slab.rollback(S, acc, *(inp[n] for n in NAMES))
    for u in range(N):
        Su = S0[u:u + 1].clone()
        for m in range(acc[u]):
            gdn.step(Su, *(inp[n][m, u:u + 1].contiguous() for n in NAMES))
        assert bits_equal(host(S[u:u + 1]), host(Su)), u
    z = torch.randn((M, N, vh, vd), generator=gen, device="cuda")
    w = torch.ones((vd,), device="cuda")
    Sg = S0.clone()
    out = gdn.step_gated(Sg, *(inp[n] for n in NAMES), z, w, 1e-6)
    assert bits_equal(host(Sg), host(S1))
    Sg1 = S0.clone()
    for m in range(M):
        og = gdn.step_gated(Sg1, *(inp[n][m:m + 1].contiguous() for n in NAMES),
                            z[m:m + 1].contiguous(), w, 1e-6)
        assert bits_equal(host(og[0]), host(out[m])), m


def test_rollback_state_only_and_zero_accept():
    dims = synth.DIMS128
    N, M = 4, 3
    gen = synth.make_gen(7, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    S_mark = S.clone()
    slab = gdn.Slab(N, dims)
    slab.mark(S)
    gdn.step_m(S, *(inp[n] for n in NAMES))
    slab.rollback(S, [0] * N, M=M)                 # no inputs needed for a pure restore
    assert bits_equal(host(S), host(S_mark))
    # the history cannot be rolled back when it was not marked
    slab.mark(S)
    with pytest.raises(gdn.GdnError):
        slab.rollback(S, [0] * N, M=M, hist=torch.zeros((N, 3, 10240), device="cuda"),
                      xc_raw=torch.zeros((M, N, 10240), device="cuda"))


# ---------------------------------------------------------------------------
# front end
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dims,B,dim", [
    (synth.DIMS128, 13, 5120),       # ragged against 8-row GEMV tiles
    (synth.DIMS64, 9, 5120),
    ((6, 2, 64, 64), 3, 100),        # conv_dim 640 < one 1024-channel block; dim not /1024
    ((6, 3, 128, 128), 1, 2052),
])
def test_frontend_parity(orc, dims, B, dim):
    say(f"frontend dims={dims} B={B} dim={dim}")
    vh, kh, kd, vd = dims
    gen = synth.make_gen(8, "cuda")
    w = synth.frontend_weights(gen, dims, dim=dim, device="cuda")
    fe = synth.frontend_inputs(gen, B, dims, T=2, dim=dim, device="cuda")
    hist = fe["hist"]
    hist_h = host(hist)
    wh = {n: host(t) for n, t in w.items()}
    for t in range(2):
        x, xc = fe["x"][t], fe["xc_raw"][t]
        out = gdn.frontend(x, w["Wa"], w["Wb"], w["A_log"], w["dt_bias"], xc, hist,
                           w["conv_w"], dims)
        ref = dict(q=np.zeros((B, kh, kd), np.float32), k=np.zeros((B, kh, kd), np.float32),
                   v=np.zeros((B, vh, vd), np.float32), g=np.zeros((B, vh), np.float32),
                   beta=np.zeros((B, vh), np.float32))
        orc.gdn_frontend(host(x), wh["Wa"], wh["Wb"], wh["A_log"], wh["dt_bias"], host(xc),
                         hist_h, wh["conv_w"], ref["q"], ref["k"], ref["v"], ref["g"],
                         ref["beta"], dims)
        for n in NAMES:
            assert_close(host(out[n]), ref[n], f"{n} t={t}")
        assert bits_equal(host(hist), hist_h)


@pytest.mark.parametrize("dims,B", [(synth.DIMS128, 5), (synth.DIMS128, 13), (synth.DIMS64, 3)])
def test_frontend_nan_stays_in_its_sequence(orc, dims, B):
    """A NaN in one sequence's hidden input x, and another in one raw conv
    channel of a second sequence: the NaN positions of q, k, v, g, beta and
    the history equal the oracle's, the finite elements agree within
    tolerance, and the other sequences keep the bits of the NaN-free call."""
    say(f"frontend NaN isolation dims={dims} B={B}")
    vh, kh, kd, vd = dims
    gen = synth.make_gen(23, "cuda")
    w = synth.frontend_weights(gen, dims, device="cuda")
    fe = synth.frontend_inputs(gen, B, dims, T=1, device="cuda")
    x, xc, h0 = fe["x"][0], fe["xc_raw"][0], fe["hist"]
    hist_c = h0.clone()
    clean = gdn.frontend(x, w["Wa"], w["Wb"], w["A_log"], w["dt_bias"], xc, hist_c,
                         w["conv_w"], dims)
    clean = {n: host(t) for n, t in clean.items()}
    bx, bc = 1, B - 1
    x, xc = x.clone(), xc.clone()
    x[bx, 17] = float("nan")
    xc[bc, kh * kd + 5] = float("nan")             # a channel of the k part
    hist = h0.clone()
    out = gdn.frontend(x, w["Wa"], w["Wb"], w["A_log"], w["dt_bias"], xc, hist, w["conv_w"],
                       dims)
    wh = {n: host(t) for n, t in w.items()}
    ref = dict(q=np.zeros((B, kh, kd), np.float32), k=np.zeros((B, kh, kd), np.float32),
               v=np.zeros((B, vh, vd), np.float32), g=np.zeros((B, vh), np.float32),
               beta=np.zeros((B, vh), np.float32))
    hist_h = host(h0)
    orc.gdn_frontend(host(x), wh["Wa"], wh["Wb"], wh["A_log"], wh["dt_bias"], host(xc), hist_h,
                     wh["conv_w"], ref["q"], ref["k"], ref["v"], ref["g"], ref["beta"], dims)
    any_nan = False
    for n in NAMES:
        got, r = host(out[n]), ref[n]
        nan = np.isnan(r)
        any_nan |= bool(nan.any())
        assert np.array_equal(np.isnan(got), nan), n
        assert_close(got[~nan], r[~nan], n)
        keep = [b for b in range(B) if b not in (bx, bc)]
        assert bits_equal(got[keep], clean[n][keep]), n
    assert any_nan
    assert np.array_equal(np.isnan(host(hist)), np.isnan(hist_h))


@pytest.mark.parametrize("dims,B,M", [(synth.DIMS128, 5, 3), (synth.DIMS64, 3, 8),
                                      (synth.DIMS128, 2, 1), (synth.DIMS128, 1, 8),
                                      (synth.DIMS64, 1, 3), (synth.DIMS128, 1, 12),
                                      (synth.DIMS128, 3, 3), (synth.DIMS128, 9, 3),
                                      (synth.DIMS64, 10, 2), (synth.DIMS128, 4, 2)])
def test_frontend_m_bit_exact_and_parity(orc, dims, B, M):
    """M draft rows in one call == M single-row GPU calls (bit for bit), and
    the oracle's M-row front end within tolerance (history bit for bit).  The
    GEMV has three shapes (one row; 2 to 8 rows; more), and the cases pair
    each with the others: B = 1 against M = 3, 8 (2-8 rows) and 12 (more), B
    = 3 or 5 (2-8 rows) against 9 or 15 rows (more, the first ragged).
    The conv of an M-row call runs its rows in parallel up to 8 sequences and
    slides one window per sequence beyond (B = 9, 10), as single-row calls
    always do."""
    say(f"frontend_m dims={dims} B={B} M={M}")
    vh, kh, kd, vd = dims
    gen = synth.make_gen(9, "cuda")
    w = synth.frontend_weights(gen, dims, device="cuda")
    fe = synth.frontend_inputs(gen, B, dims, T=M, device="cuda")
    h0 = fe["hist"].clone()
    hist_m = fe["hist"].clone()
    out_m = gdn.frontend_m(fe["x"], w["Wa"], w["Wb"], w["A_log"], w["dt_bias"], fe["xc_raw"],
                           hist_m, w["conv_w"], dims)
    hist_1 = h0.clone()
    for m in range(M):
        one = gdn.frontend(fe["x"][m], w["Wa"], w["Wb"], w["A_log"], w["dt_bias"],
                           fe["xc_raw"][m], hist_1, w["conv_w"], dims)
        for n in NAMES:
            assert bits_equal(host(out_m[n][m]), host(one[n])), (n, m)
    assert bits_equal(host(hist_m), host(hist_1))
    wh = {n: host(t) for n, t in w.items()}
    ref = dict(q=np.zeros((M, B, kh, kd), np.float32), k=np.zeros((M, B, kh, kd), np.float32),
               v=np.zeros((M, B, vh, vd), np.float32), g=np.zeros((M, B, vh), np.float32),
               beta=np.zeros((M, B, vh), np.float32))
    h_ref = host(h0)
    orc.gdn_frontend_m(host(fe["x"]), wh["Wa"], wh["Wb"], wh["A_log"], wh["dt_bias"],
                       host(fe["xc_raw"]), h_ref, wh["conv_w"], ref["q"], ref["k"], ref["v"],
                       ref["g"], ref["beta"], dims)
    for n in NAMES:
        assert_close(host(out_m[n]), ref[n], f"frontend_m {n}")
    assert bits_equal(host(hist_m), h_ref)


@pytest.mark.parametrize("dims,dim", [(synth.DIMS128, 5120), (synth.DIMS64, 5120),
                                      ((6, 2, 64, 64), 1000), ((6, 3, 128, 128), 2052)])
def test_frontend_gemv_rows_independent_of_row_count(orc, dims, dim):
    """The paired GEMV of row r gives the same g and beta bits in calls of
    every row count, across the three GEMV shapes that serve them (one row,
    2 to 8 rows, more; the last ragged against its 8-row tiles), with dim a
    multiple of the 2048-column lane stride or not; and the oracle agrees
    within tolerance."""
    say(f"GEMV row-count independence dims={dims} dim={dim}")
    vh, kh, kd, vd = dims
    gen = synth.make_gen(23, "cuda")
    w = synth.frontend_weights(gen, dims, dim=dim, device="cuda")
    Rmax = 300
    fe = synth.frontend_inputs(gen, Rmax, dims, T=1, dim=dim, device="cuda")
    gb = {}
    for R in (1, 2, 3, 4, 5, 8, 9, 64, 128, 129, 300):
        out = gdn.frontend(fe["x"][0, :R].contiguous(), w["Wa"], w["Wb"], w["A_log"],
                           w["dt_bias"], fe["xc_raw"][0, :R].contiguous(),
                           fe["hist"][:R].clone(), w["conv_w"], dims)
        gb[R] = (host(out["g"]), host(out["beta"]))
    for R, (g_, b_) in gb.items():
        n = min(R, 64)
        assert bits_equal(g_[:n], gb[300][0][:n]) and bits_equal(b_[:n], gb[300][1][:n]), R
        assert bits_equal(g_[:1], gb[1][0]) and bits_equal(b_[:1], gb[1][1]), R
    wh = {n: host(t) for n, t in w.items()}
    R = 9
    ref = dict(q=np.zeros((R, kh, kd), np.float32), k=np.zeros((R, kh, kd), np.float32),
               v=np.zeros((R, vh, vd), np.float32), g=np.zeros((R, vh), np.float32),
               beta=np.zeros((R, vh), np.float32))
    orc.gdn_frontend(host(fe["x"][0, :R]), wh["Wa"], wh["Wb"], wh["A_log"], wh["dt_bias"],
                     host(fe["xc_raw"][0, :R]), host(fe["hist"][:R]), wh["conv_w"], ref["q"],
                     ref["k"], ref["v"], ref["g"], ref["beta"], dims)
    assert_close(gb[9][0], ref["g"], "g")
    assert_close(gb[9][1], ref["beta"], "beta")


def test_verify_cycle_with_frontend(orc):
    """mark(S, hist) -> frontend_m -> step_m -> rollback(S, hist): the whole
    speculative-verify chain of one layer against the oracle's chain."""
    dims = synth.DIMS128
    vh, kh, kd, vd = dims
    B, M = 6, 4
    cd = synth.conv_dim_of(dims)
    gen = synth.make_gen(10, "cuda")
    S = synth.state(gen, B, dims, device="cuda")
    w = synth.frontend_weights(gen, dims, device="cuda")
    fe = synth.frontend_inputs(gen, B, dims, T=M, device="cuda")
    hist = fe["hist"]
    S_h, hist_h = host(S), host(hist)
    acc = [0, 1, 4, 2, 3, 4]
    slab = gdn.Slab(B, dims, hist_floats_per_unit=3 * cd)
    slab.mark(S, hist)
    rows = gdn.frontend_m(fe["x"], w["Wa"], w["Wb"], w["A_log"], w["dt_bias"], fe["xc_raw"],
                          hist, w["conv_w"], dims)
    o = gdn.step_m(S, *(rows[n] for n in NAMES))
    slab.rollback(S, acc, *(rows[n] for n in NAMES), hist=hist, xc_raw=fe["xc_raw"])
    # oracle chain
    wh = {n: host(t) for n, t in w.items()}
    ref = dict(q=np.zeros((M, B, kh, kd), np.float32), k=np.zeros((M, B, kh, kd), np.float32),
               v=np.zeros((M, B, vh, vd), np.float32), g=np.zeros((M, B, vh), np.float32),
               beta=np.zeros((M, B, vh), np.float32))
    rs = orc.slab(B, dims, hist_floats=3 * cd)
    rs.mark(S_h, hist_h)
    orc.gdn_frontend_m(host(fe["x"]), wh["Wa"], wh["Wb"], wh["A_log"], wh["dt_bias"],
                       host(fe["xc_raw"]), hist_h, wh["conv_w"], ref["q"], ref["k"], ref["v"],
                       ref["g"], ref["beta"], dims)
    o_ref = np.zeros((M, B, vh, vd), np.float32)
    orc.gdn_step_m(S_h, *(ref[n] for n in NAMES), o_ref, M, dims)
    assert_close(host(o), o_ref, "o verify")
    rs.rollback(S_h, hist_h, ref, M, np.array(acc, np.int32), xc_raw=host(fe["xc_raw"]),
                conv_dim=cd, ck=4)
    assert_close(host(S), S_h, "S after rollback")
    assert bits_equal(host(hist), hist_h)


@pytest.mark.parametrize("dims,M", [(synth.DIMS128, 1), (synth.DIMS128, 5), (synth.DIMS64, 1),
                                    (synth.DIMS64, 3)])
def test_step_gated_parity(orc, dims, M):
    """Gated RMSNorm fused on the output: the state advances exactly as in
    the ungated call (bits); the output matches the oracle's step followed by
    the oracle's gated norm; M rows equal M single gated steps (bits)."""
    say(f"step_gated dims={dims} M={M}")
    vh, kh, kd, vd = dims
    N = 4
    gen = synth.make_gen(12, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    z = torch.randn((M, N, vh, vd), generator=gen, device="cuda")
    w = 1.0 + 0.1 * torch.randn((vd,), generator=gen, device="cuda")
    eps = 1e-6
    S_plain = S.clone()
    S_h = host(S)
    out = gdn.step_gated(S, *(inp[n] for n in NAMES), z, w, eps)
    if M == 1:
        o_plain = gdn.step(S_plain, *(inp[n][0] for n in NAMES)).unsqueeze(0)
    else:
        o_plain = gdn.step_m(S_plain, *(inp[n] for n in NAMES))
    assert bits_equal(host(S), host(S_plain))
    # the epilogue alone, at o's own bound: the gated kernel forms the same
    # raw o as the ungated call (the same canonical tree), so its output is
    # the oracle's gated norm of that o up to the norm's own rounding
    g_own = np.zeros((M, N, vh, vd), np.float32)
    orc.gated_norm(host(o_plain), host(z), host(w), eps, g_own)
    assert_close(host(out), g_own, "gated epilogue on the GPU's o", rel=1e-5, floor=1e-6)
    o_ref = np.zeros((M, N, vh, vd), np.float32)
    orc.gdn_step_m(S_h, *(host(inp[n]) for n in NAMES), o_ref, M, dims)
    g_ref = np.zeros_like(o_ref)
    orc.gated_norm(o_ref, host(z), host(w), eps, g_ref)
    # out = o * s with s = w * silu(z) / sqrt(mean(o^2) + eps): o's tolerance
    # (1e-5 relative, 1e-6 absolute) carries over, its absolute floor scaled by s
    o64, z64 = o_ref.astype(np.float64), host(z).astype(np.float64)
    rinv = 1.0 / np.sqrt(np.mean(o64 ** 2, axis=-1, keepdims=True) + eps)
    scale = np.abs(rinv * host(w).astype(np.float64) * z64 / (1.0 + np.exp(-z64)))
    assert_close(host(out), g_ref, "gated out", rel=1e-5, floor=1e-6 * scale)
    if M > 1:
        S1 = synth.state(synth.make_gen(12, "cuda"), N, dims, device="cuda")
        for m in range(M):
            o1 = gdn.step_gated(S1, *(inp[n][m:m + 1].contiguous() for n in NAMES),
                                z[m:m + 1].contiguous(), w, eps)
            assert bits_equal(host(o1[0]), host(out[m])), m


@pytest.mark.parametrize("dims,M", [(synth.DIMS128, 1), (synth.DIMS128, 5), (synth.DIMS128, 10),
                                    (synth.DIMS64, 1), (synth.DIMS64, 6)])
def test_verify_m_gated_equals_step_gated(orc, dims, M):
    """gdn_verify_m_gated gives the outputs of gdn_step_gated bit for bit
    (single-step, M-step and prefetching instances) and leaves S untouched."""
    say(f"verify_m_gated dims={dims} M={M}")
    vh, kh, kd, vd = dims
    N = 3
    gen = synth.make_gen(14, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    z = torch.randn((M, N, vh, vd), generator=gen, device="cuda")
    w = 1.0 + 0.1 * torch.randn((vd,), generator=gen, device="cuda")
    S0 = host(S)
    out_v = gdn.verify_m_gated(S, *(inp[n] for n in NAMES), z, w, 1e-6)
    assert bits_equal(host(S), S0)
    out_s = gdn.step_gated(S.clone(), *(inp[n] for n in NAMES), z, w, 1e-6)
    assert bits_equal(host(out_v), host(out_s))
    o_ref = np.zeros((M, N, vh, vd), np.float32)
    orc.gdn_step_m(S0.copy(), *(host(inp[n]) for n in NAMES), o_ref, M, dims)
    g_ref, g_floor = ref_gated(orc, o_ref, host(z), host(w), 1e-6)
    assert_close(host(out_v), g_ref, "verify_m_gated out", floor=g_floor)
    # the epilogue at o's own bound, on the GPU's raw o of the same rows
    o_gpu = gdn.verify_m(S, *(inp[n] for n in NAMES))
    g_own = np.zeros_like(o_ref)
    orc.gated_norm(host(o_gpu), host(z), host(w), 1e-6, g_own)
    assert_close(host(out_v), g_own, "verify_m_gated epilogue on the GPU's o", rel=1e-5,
                 floor=1e-6)


@pytest.mark.parametrize("dims", [synth.DIMS128, synth.DIMS64])
def test_verify_commit_equals_snapshot_protocol(orc, dims):
    """verify_m + commit(accepted) gives the same outputs, state and conv
    history, bit for bit, as mark + step_m + rollback(accepted); verify_m
    leaves the state untouched."""
    say(f"verify/commit dims={dims}")
    vh, kh, kd, vd = dims
    N, M = 6, 5
    cd = synth.conv_dim_of(dims)
    gen = synth.make_gen(15, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    hist = torch.randn((N, 3, cd), generator=gen, device="cuda")
    xc = torch.randn((M, N, cd), generator=gen, device="cuda")
    acc = [0, 1, 2, M, 3, 4]
    args = [inp[n] for n in NAMES]
    # snapshot protocol
    S_a, h_a = S.clone(), hist.clone()
    slab = gdn.Slab(N, dims, hist_floats_per_unit=3 * cd)
    slab.mark(S_a, h_a)
    o_a = gdn.step_m(S_a, *args)
    slab.rollback(S_a, acc, *args, hist=h_a, xc_raw=xc)
    # verify / commit protocol
    S_b, h_b = S.clone(), hist.clone()
    o_b = gdn.verify_m(S_b, *args)
    assert bits_equal(host(S_b), host(S))
    acc_dev = torch.tensor(acc, dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gdn.commit(S_b, acc_dev, *args, hist=h_b, xc_raw=xc, status=status)
    assert bits_equal(host(o_a), host(o_b))
    assert bits_equal(host(S_a), host(S_b))
    assert bits_equal(host(h_a), host(h_b))
    assert int(status.item()) == 0
    # both protocols against the oracle's mark, M steps, rollback
    o_ref, _, S_rb, h_rb = ref_cycle(orc, host(S), {n: host(inp[n]) for n in NAMES}, dims, acc,
                                     host(hist), host(xc))
    assert_close(host(o_b), o_ref, "o verify_m")
    assert_close(host(S_b), S_rb, "S after commit")
    assert bits_equal(host(h_b), h_rb)


@pytest.mark.parametrize("dims", [synth.DIMS128, synth.DIMS64])
def test_single_row_commit_and_rollback_with_history(dims):
    """M = 1: the state replay runs the single-step kernel and the history its
    own launch.  Accepted 1 equals one step and one pushed frame; accepted 0
    leaves state and history as they were (bit for bit, both entry points)."""
    say(f"M=1 commit/rollback with history dims={dims}")
    vh, kh, kd, vd = dims
    N, conv_dim = 5, synth.conv_dim_of(dims)
    gen = synth.make_gen(63, "cuda")
    S0 = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=1, device="cuda")
    h0 = torch.randn((N, 3, conv_dim), generator=gen, device="cuda")
    xc = torch.randn((1, N, conv_dim), generator=gen, device="cuda")
    acc = [1, 0, 1, 1, 0]
    S1 = S0.clone()
    gdn.step(S1, *(inp[n][0] for n in NAMES))
    S_want = torch.stack([S1[u] if a else S0[u] for u, a in enumerate(acc)])
    h_want = torch.stack([torch.cat([h0[u, 1:], xc[0, u:u + 1]]) if a else h0[u]
                          for u, a in enumerate(acc)])
    S_c, h_c = S0.clone(), h0.clone()
    gdn.commit(S_c, torch.tensor(acc, dtype=torch.int32, device="cuda"),
               *(inp[n] for n in NAMES), hist=h_c, xc_raw=xc)
    assert bits_equal(host(S_c), host(S_want)) and bits_equal(host(h_c), host(h_want))
    slab = gdn.Slab(N, dims, hist_floats_per_unit=3 * conv_dim)
    S_r, h_r = S0.clone(), h0.clone()
    slab.mark(S_r, hist=h_r)
    gdn.step(S_r, *(inp[n][0] for n in NAMES))
    h_r.normal_(generator=gen)                     # clobbered, restored by the rollback
    slab.rollback(S_r, acc, *(inp[n] for n in NAMES), hist=h_r, xc_raw=xc)
    assert bits_equal(host(S_r), host(S_want)) and bits_equal(host(h_r), host(h_want))


def test_commit_refuses_out_of_range_counts(orc):
    """Device-supplied counts outside 0..M leave that unit unchanged and raise
    the status flag; the other units are committed normally."""
    dims = synth.DIMS128
    N, M = 4, 3
    cd = synth.conv_dim_of(dims)
    gen = synth.make_gen(16, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    hist = torch.randn((N, 3, cd), generator=gen, device="cuda")
    xc = torch.randn((M, N, cd), generator=gen, device="cuda")
    S0, h0 = S.clone(), hist.clone()
    acc = torch.tensor([1, M + 1, -1, 2], dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gdn.commit(S, acc, *(inp[n] for n in NAMES), hist=hist, xc_raw=xc, status=status)
    assert int(status.item()) == 1
    for u in (1, 2):
        assert bits_equal(host(S[u]), host(S0[u])) and bits_equal(host(hist[u]), host(h0[u]))
    for u, a in ((0, 1), (3, 2)):
        Su = S0[u:u + 1].clone()
        for m in range(a):
            gdn.step(Su, *(inp[n][m, u:u + 1].contiguous() for n in NAMES))
        assert bits_equal(host(S[u:u + 1]), host(Su)), u
        seq = np.concatenate([host(h0[u]), host(xc[:a, u])], axis=0)
        assert bits_equal(host(hist[u]), seq[-3:]), u
    # the oracle refuses such counts outright; the units it can take (the
    # in-range ones, refused ones as accepted = 0) give the same result
    _, _, S_rb, h_rb = ref_cycle(orc, host(S0), {n: host(inp[n]) for n in NAMES}, dims,
                                 [1, 0, 0, 2], host(h0), host(xc))
    assert_close(host(S), S_rb, "S after commit")
    assert bits_equal(host(hist), h_rb)


def test_commit_single_step_history_beyond_65536_units(orc):
    """A one-step commit with a history replays it in a launch of its own; its
    grid holds every unit in one dimension, so more than 65536 units (one key
    and one value head of kd = 64 each: 1 GB of state) are all committed.
    Checked against the oracle's cycle: S within tolerance, the history bit
    for bit, refused counts leaving their unit unchanged."""
    dims = (1, 1, 64, 64)
    N, M = 65536 + 37, 1
    say(f"commit M=1 with history, N={N} dims={dims}")
    cd = synth.conv_dim_of(dims)
    gen = synth.make_gen(17, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    hist = torch.randn((N, 3, cd), generator=gen, device="cuda")
    xc = torch.randn((M, N, cd), generator=gen, device="cuda")
    S0, h0 = host(S), host(hist)
    acc = (torch.arange(N, device="cuda") % 2).to(torch.int32)
    acc[-1] = 2                                   # out of range: this unit stays
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gdn.commit(S, acc, *(inp[n] for n in NAMES), hist=hist, xc_raw=xc, status=status)
    assert int(status.item()) == 1
    acc_ref = host(acc).copy()
    acc_ref[-1] = 0
    _, _, S_rb, h_rb = ref_cycle(orc, S0, {n: host(inp[n]) for n in NAMES}, dims, acc_ref, h0,
                                 host(xc))
    assert_close(host(S), S_rb, "S after commit")
    assert bits_equal(host(hist), h_rb)
    assert bits_equal(host(S[-1]), S0[-1]) and bits_equal(host(hist[-1]), h0[-1])


@pytest.mark.parametrize("dims,N,M,M2", [(synth.DIMS128, 24, 8, 8), (synth.DIMS64, 11, 3, 5),
                                         (synth.DIMS128, 24, 10, 12), (synth.DIMS128, 1, 8, 8),
                                         (synth.DIMS64, 2, 4, 4)])
def test_commit_verify_fused_equals_two_calls(orc, dims, N, M, M2):
    """gdn_commit_verify_m against gdn_commit followed by gdn_verify_m on the
    same inputs: state, history, outputs and status word bit for bit, with one
    out-of-range count (that unit keeps its state and history and still
    verifies).  1152 and 1056 tiles run the fused M-step launch (12 rows
    prefetched in one case), 48 and 192 tiles the two launches.  Then the
    oracle: the committed state is the oracle's rollback to the accepted
    rows, and the outputs its M2 steps from there."""
    say(f"commit+verify fused dims={dims} N={N} M={M} M2={M2}")
    vh, kh, kd, vd = dims
    cd = synth.conv_dim_of(dims)
    gen = synth.make_gen(18 + N, "cuda")
    S0 = synth.state(gen, N, dims, device="cuda")
    prev = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    new = synth.step_inputs(gen, N, dims, M=M2, device="cuda")
    h0 = torch.randn((N, 3, cd), generator=gen, device="cuda")
    xc = torch.randn((M, N, cd), generator=gen, device="cuda")
    acc = torch.randint(0, M + 1, (N,), generator=gen, device="cuda").to(torch.int32)
    if N > 1:
        acc[1] = M + 1                                  # refused: unit 1 stays as it is
    S_a, h_a, st_a = S0.clone(), h0.clone(), torch.zeros(1, dtype=torch.int32, device="cuda")
    o_a = gdn.commit_verify_m(S_a, acc, *(prev[n] for n in NAMES), *(new[n] for n in NAMES),
                              hist=h_a, xc_raw=xc, status=st_a)
    S_b, h_b, st_b = S0.clone(), h0.clone(), torch.zeros(1, dtype=torch.int32, device="cuda")
    gdn.commit(S_b, acc, *(prev[n] for n in NAMES), hist=h_b, xc_raw=xc, status=st_b)
    o_b = gdn.verify_m(S_b, *(new[n] for n in NAMES))
    assert bits_equal(host(S_a), host(S_b))
    assert bits_equal(host(h_a), host(h_b))
    assert bits_equal(host(o_a), host(o_b))
    assert int(st_a.item()) == int(st_b.item()) == (1 if N > 1 else 0)
    acc_ref = host(acc).copy()
    if N > 1:
        acc_ref[1] = 0
    _, _, S_rb, h_rb = ref_cycle(orc, host(S0), {n: host(prev[n]) for n in NAMES}, dims, acc_ref,
                                 host(h0), host(xc))
    assert_close(host(S_a), S_rb, "S after the fused commit")
    assert bits_equal(host(h_a), h_rb)
    o_ref = np.zeros((M2, N, vh, vd), np.float32)
    orc.gdn_step_m(S_rb.copy(), *(host(new[n]) for n in NAMES), o_ref, M2, dims)
    assert_close(host(o_a), o_ref, "o of the fused verify")


def test_commit_verify_fused_graph_replay():
    """Two steady-state cycles of the fused call (each commits the previous
    rows' accepted prefix and verifies the next rows) captured as one graph on
    the fused M-step path (1152 tiles) and replayed three times, with eager
    work between replays: state, history and both cycles' outputs equal the
    eager sequence bit for bit."""
    dims = synth.DIMS128
    vh, kh, kd, vd = dims
    N, M = 24, 4
    cd = synth.conv_dim_of(dims)
    gen = synth.make_gen(23, "cuda")
    S0 = synth.state(gen, N, dims, device="cuda")
    r1 = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    r2 = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    r3 = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    h0 = torch.randn((N, 3, cd), generator=gen, device="cuda")
    x1 = torch.randn((M, N, cd), generator=gen, device="cuda")
    x2 = torch.randn((M, N, cd), generator=gen, device="cuda")
    a1 = torch.randint(0, M + 1, (N,), generator=gen, device="cuda").to(torch.int32)
    a2 = torch.randint(0, M + 1, (N,), generator=gen, device="cuda").to(torch.int32)
    o2 = torch.empty((M, N, vh, vd), device="cuda")
    o3 = torch.empty((M, N, vh, vd), device="cuda")
    S, hist = S0.clone(), h0.clone()

    def cycles():
        gdn.commit_verify_m(S, a1, *(r1[n] for n in NAMES), *(r2[n] for n in NAMES), o=o2,
                            hist=hist, xc_raw=x1)
        gdn.commit_verify_m(S, a2, *(r2[n] for n in NAMES), *(r3[n] for n in NAMES), o=o3,
                            hist=hist, xc_raw=x2)

    cycles()
    torch.cuda.synchronize()
    S_e, h_e, o2_e, o3_e = host(S), host(hist), host(o2), host(o3)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        S.copy_(S0)
        hist.copy_(h0)
        cycles()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cycles()
    for rep in range(3):
        S.copy_(S0)
        hist.copy_(h0)
        o2.zero_()
        o3.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert bits_equal(host(S), S_e) and bits_equal(host(hist), h_e), rep
        assert bits_equal(host(o2), o2_e) and bits_equal(host(o3), o3_e), rep
        gdn.step(S0.clone(), *(r1[n][0] for n in NAMES))   # eager work between replays


def test_verify_cycle_graph_replay(orc):
    """One layer's speculative cycle without a snapshot -- front end for the M
    draft rows (history read only), verify, commit with device-side accepted
    lengths -- captured as a graph and replayed three times against eager
    execution of the same cycle, bit for bit."""
    dims = synth.DIMS128
    vh, kh, kd, vd = dims
    B, M = 4, 3
    gen = synth.make_gen(17, "cuda")
    S0 = synth.state(gen, B, dims, device="cuda")
    w = synth.frontend_weights(gen, dims, device="cuda")
    fe = synth.frontend_inputs(gen, B, dims, T=M, device="cuda")
    h0 = fe["hist"].clone()
    acc = torch.tensor([3, 0, 1, 2], dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    rows = dict(q=torch.empty((M, B, kh, kd), device="cuda"),
                k=torch.empty((M, B, kh, kd), device="cuda"),
                v=torch.empty((M, B, vh, vd), device="cuda"),
                g=torch.empty((M, B, vh), device="cuda"),
                beta=torch.empty((M, B, vh), device="cuda"))
    o = torch.empty((M, B, vh, vd), device="cuda")
    S, hist = S0.clone(), h0.clone()

    def cycle():
        gdn.frontend_verify_m(fe["x"], w["Wa"], w["Wb"], w["A_log"], w["dt_bias"], fe["xc_raw"],
                              hist, w["conv_w"], dims, out=rows)
        gdn.verify_m(S, *(rows[n] for n in NAMES), o=o)
        gdn.commit(S, acc, *(rows[n] for n in NAMES), hist=hist, xc_raw=fe["xc_raw"],
                   status=status)

    cycle()
    torch.cuda.synchronize()
    S_e, h_e, o_e = host(S), host(hist), host(o)
    # the eager cycle agrees with the snapshot protocol driven by frontend_m
    S_s, h_s = S0.clone(), h0.clone()
    slab = gdn.Slab(B, dims, hist_floats_per_unit=3 * synth.conv_dim_of(dims))
    slab.mark(S_s, h_s)
    rows_s = gdn.frontend_m(fe["x"], w["Wa"], w["Wb"], w["A_log"], w["dt_bias"], fe["xc_raw"],
                            h_s, w["conv_w"], dims)
    o_s = gdn.step_m(S_s, *(rows_s[n] for n in NAMES))
    slab.rollback(S_s, host(acc), *(rows_s[n] for n in NAMES), hist=h_s, xc_raw=fe["xc_raw"])
    assert bits_equal(host(S_s), S_e) and bits_equal(host(h_s), h_e) and bits_equal(host(o_s), o_e)
    # the cycle against the oracle's chain: mark, frontend_m, step_m, rollback
    wh = {n: host(t) for n, t in w.items()}
    ref = dict(q=np.zeros((M, B, kh, kd), np.float32), k=np.zeros((M, B, kh, kd), np.float32),
               v=np.zeros((M, B, vh, vd), np.float32), g=np.zeros((M, B, vh), np.float32),
               beta=np.zeros((M, B, vh), np.float32))
    h_fe = host(h0)
    orc.gdn_frontend_m(host(fe["x"]), wh["Wa"], wh["Wb"], wh["A_log"], wh["dt_bias"],
                       host(fe["xc_raw"]), h_fe, wh["conv_w"], ref["q"], ref["k"], ref["v"],
                       ref["g"], ref["beta"], dims)
    o_ref, _, S_rb, h_rb = ref_cycle(orc, host(S0), ref, dims, host(acc), host(h0),
                                     host(fe["xc_raw"]))
    assert_close(o_e, o_ref, "o verify cycle")
    assert_close(S_e, S_rb, "S verify cycle")
    assert bits_equal(h_e, h_rb)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        S.copy_(S0)
        hist.copy_(h0)
        cycle()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cycle()
    for rep in range(3):
        S.copy_(S0)
        hist.copy_(h0)
        o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert bits_equal(host(S), S_e) and bits_equal(host(hist), h_e), rep
        assert bits_equal(host(o), o_e), rep
        gdn.step(S0.clone(), *(rows[n][0] for n in NAMES))   # eager work between replays
        torch.cuda.synchronize()
    assert int(status.item()) == 0
    del graph


def test_graph_replay_matches_eager(orc):
    """A captured chain of 8 single steps (the per-token launch chain) replays
    bit-identically to eager execution, several times, with eager work and
    synchronisations between the replays.  The captured path records kernel
    launches only (no memset nodes)."""
    dims = synth.DIMS128
    N, T = 2, 8
    gen = synth.make_gen(11, "cuda")
    S0 = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=T, device="cuda")
    rows = [{n: inp[n][m] for n in NAMES} for m in range(T)]
    S_e = S0.clone()
    o_e = [gdn.step(S_e, *(x[n] for n in NAMES)) for x in rows]
    torch.cuda.synchronize()
    S_ref = host(S0)
    o_ref = ref_steps(orc, S_ref, {n: host(inp[n]) for n in NAMES}, dims, T)
    for m in range(T):
        assert_close(host(o_e[m]), o_ref[m], f"o step {m}")
    assert_close(host(S_e), S_ref, "S after the chain")
    S_g = S0.clone()
    outs = [torch.empty((N, dims[0], dims[3]), device="cuda") for _ in range(T)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):              # warm-up outside capture
        for x, o in zip(rows, outs):
            gdn.step(S_g, *(x[n] for n in NAMES), o=o)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for x, o in zip(rows, outs):
            gdn.step(S_g, *(x[n] for n in NAMES), o=o)
    for rep in range(3):
        S_g.copy_(S0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert bits_equal(host(S_g), host(S_e)), rep
        for m in range(T):
            assert bits_equal(host(outs[m]), host(o_e[m])), (rep, m)
        S_tmp = S0.clone()                         # eager work between replays
        gdn.step(S_tmp, *(rows[0][n] for n in NAMES))
        torch.cuda.synchronize()
    del graph


def test_zero_sized_calls_are_no_ops():
    dims = synth.DIMS128
    vh, kh, kd, vd = dims
    e = torch.empty(0, device="cuda")
    L = gdn.lib()
    st = torch.cuda.current_stream().cuda_stream
    P = lambda t: C.c_void_p(t.data_ptr())  # noqa: E731
    assert L.gdn_step(P(e), P(e), P(e), P(e), P(e), P(e), P(e), 0, vh, kh, kd, vd,
                      C.c_void_p(st)) == 0
    assert L.gdn_frontend(*([P(e)] * 13), 0, 5120, synth.conv_dim_of(dims), 4, vh, kh, kd, vd,
                          C.c_void_p(st)) == 0
    torch.cuda.synchronize()


def test_stream_read_words():
    """The read-only floor's chunk checksums equal the XOR of each 128 KiB
    chunk's words, for sizes with a ragged last chunk and a 1..3-float tail."""
    for n in (1, 3, 4, 32768, 32769, 32768 * 5 + 7, 1000003):
        src = torch.randn(n, device="cuda")
        words = gdn.stream_read(src)
        x = host(src).view(np.uint32)
        nc = (n + 32767) // 32768
        want = np.array([np.bitwise_xor.reduce(x[32768 * c:32768 * (c + 1)]) for c in range(nc)],
                        np.uint32)
        assert words.numel() == nc, n
        assert bits_equal(host(words).view(np.uint32), want), n


def test_stream_copy_ragged():
    for n in (1, 3, 4, 1000003, 4 * 256 * 4 * 3 + 5):
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        gdn.stream_copy(dst, src)
        assert bits_equal(host(dst), host(src)), n
        gdn.stream_copy(src, src)                  # in place: read and write back
        assert bits_equal(host(dst), host(src)), n


def test_binding_refuses_mis_sized_tensors():
    """The binding checks every tensor's element count before calling the C
    ABI (which receives raw pointers): a short or long buffer is refused with
    ValueError and nothing is launched."""
    dims = synth.DIMS128
    vh, kh, kd, vd = dims
    N, M = 2, 3
    gen = synth.make_gen(15, "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    S0 = host(S)
    row = [inp[n][0] for n in NAMES]
    for i, name in enumerate(NAMES):
        bad = list(row)
        bad[i] = bad[i].reshape(-1)[:-4].contiguous()          # 4 elements short
        with pytest.raises(ValueError, match=name):
            gdn.step(S, *bad)
    with pytest.raises(ValueError, match="o"):
        gdn.step(S, *row, o=torch.empty((N, vh, vd - 4), device="cuda"))
    with pytest.raises(ValueError, match="v"):
        gdn.step_m(S, *(inp[n] for n in NAMES[:2]), inp["v"][:2].contiguous(), inp["g"],
                   inp["beta"])
    with pytest.raises(ValueError, match="accepted"):
        gdn.commit(S, torch.zeros(N + 1, dtype=torch.int32, device="cuda"),
                   *(inp[n] for n in NAMES))
    w = synth.frontend_weights(gen, dims, dim=256, device="cuda")
    fe = synth.frontend_inputs(gen, N, dims, dim=256, device="cuda")
    with pytest.raises(ValueError, match="hist"):
        gdn.frontend(fe["x"][0], w["Wa"], w["Wb"], w["A_log"], w["dt_bias"], fe["xc_raw"][0],
                     fe["hist"][:1].contiguous(), w["conv_w"], dims)
    torch.cuda.synchronize()
    assert bits_equal(host(S), S0)
