"""GPU parity at the workloads' full sizes, on every unit.

Each test runs one workload in the launch configuration the benchmark times
(one launch over all units per call), keeps what the GPU produced on the
device, and then recomputes every unit with the oracle on a pool of host
threads, a range of units at a time (units are independent, so a range is
exact), comparing per element with |x - r| <= max(1e-5 |r|, 1e-6).  Host
memory stays bounded by the ranges in flight.  Bit-exact checks (between the
two speculative protocols, rollback(0), rollback(M)) run on the device.
The pages check every element of a layer the same way ("Kestrel_VLLM #24",
section 7: layer 0 against layer 47, no element differing).
"""
import numpy as np
import pytest
import torch

import gated_deltanet_recurrent_amd as gdn
import synth
from tests.helpers import Tally, over_unit_chunks

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


def same_bits(a, b):
    """Bit equality of two device tensors, on the device."""
    return a.shape == b.shape and torch.equal(a.reshape(-1).view(torch.int32),
                                              b.reshape(-1).view(torch.int32))


def merge(results):
    out = [Tally() for _ in results[0]]
    for r in results:
        for t, x in zip(out, r):
            t.merge(x)
    return out


@pytest.mark.timeout(900)
@pytest.mark.parametrize("wl,T", [(1, 3), (4, 50), (5, 50)])
def test_full_size_steps_every_unit(orc, wl, T):
    """Decode steps over all units: workload 1 (64 x 48 units) for 3 steps,
    workloads 4 and 5 (512 x 8 units, slow decay alpha in [0.5, 1]) for all
    50 chained steps; o of every step, S after the first and the last step."""
    cfg = synth.WORKLOADS[wl]
    dims = cfg["dims"]
    vh, kh, kd, vd = dims
    N = cfg["seqs"] * cfg["layers"]
    say(f"full size, every unit: {cfg['name']}: {N} units x {T} steps")
    gen = synth.make_gen(cfg["seed"], "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=T, gate=cfg["gate"], device="cuda")
    S0 = S.clone()
    O = torch.empty((T, N, vh, vd), device="cuda")
    S1 = None
    for t in range(T):
        gdn.step(S, *(inp[n][t] for n in NAMES), o=O[t])
        if t == 0:
            S1 = S.clone()
    torch.cuda.synchronize()
    assert torch.isfinite(O).all() and torch.isfinite(S).all()

    def check(lo, hi):
        to, ts = Tally(), Tally()
        S_h = host(S0[lo:hi])
        x_h = {n: host(inp[n][:, lo:hi]) for n in NAMES}
        O_h = host(O[:, lo:hi])
        o_ref = np.zeros((hi - lo, vh, vd), np.float32)
        for t in range(T):
            orc.gdn_step(S_h, *(np.ascontiguousarray(x_h[n][t]) for n in NAMES), o_ref, dims)
            to.add(O_h[t], o_ref)
            if t == 0:
                ts.add(host(S1[lo:hi]), S_h)
        ts.add(host(S[lo:hi]), S_h)
        return to, ts

    to, ts = merge(over_unit_chunks(check, N, 32))
    say(f"  o: {to}; S: {ts}")
    assert to.n == T * N * vh * vd and ts.n == 2 * N * vh * kd * vd
    assert to.bad == 0 and ts.bad == 0


@pytest.mark.timeout(900)
def test_full_size_verify_cycle_every_unit(orc):
    """Workload 2 (32 x 48 units, M = 8 draft rows, accepted lengths drawn per
    sequence and shared by its 48 layers) in both protocols: mark, step_m,
    rollback; and verify_m, commit (device-side counts).  The two agree bit
    for bit on the device; every unit's outputs, M-step state and final state
    against the oracle's mark, M steps, rollback."""
    cfg = synth.WORKLOADS[2]
    dims = cfg["dims"]
    vh, kh, kd, vd = dims
    L, M = cfg["layers"], cfg["M"]
    N = cfg["seqs"] * L
    say(f"full size, every unit: {cfg['name']}: {N} units, M = {M}")
    gen = synth.make_gen(cfg["seed"], "cuda")
    S = synth.state(gen, N, dims, device="cuda")
    inp = synth.step_inputs(gen, N, dims, M=M, device="cuda")
    rng = np.random.default_rng(2)
    acc = np.repeat(rng.integers(0, M + 1, cfg["seqs"]), L).astype(np.int32)
    S0 = S.clone()
    # snapshot protocol
    slab = gdn.Slab(N, dims)
    slab.mark(S)
    o_a = gdn.step_m(S, *(inp[n] for n in NAMES))
    S_m = S.clone()
    slab.rollback(S, acc, *(inp[n] for n in NAMES))
    del slab
    # snapshot-free protocol
    S_b = S0.clone()
    o_b = gdn.verify_m(S_b, *(inp[n] for n in NAMES))
    assert same_bits(S_b, S0)
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    gdn.commit(S_b, torch.as_tensor(acc, device="cuda"), *(inp[n] for n in NAMES), status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert same_bits(o_a, o_b) and same_bits(S, S_b)
    acc_t = torch.as_tensor(acc, device="cuda")
    assert same_bits(S[acc_t == 0], S0[acc_t == 0])
    assert same_bits(S[acc_t == M], S_m[acc_t == M])
    del S_b, o_b

    def check(lo, hi):
        to, tm, tr = Tally(), Tally(), Tally()
        S_h = host(S0[lo:hi])
        x_h = {n: host(inp[n][:, lo:hi]) for n in NAMES}
        rs = orc.slab(hi - lo, dims)
        rs.mark(S_h)
        o_ref = np.zeros((M, hi - lo, vh, vd), np.float32)
        orc.gdn_step_m(S_h, *(x_h[n] for n in NAMES), o_ref, M, dims)
        to.add(host(o_a[:, lo:hi]), o_ref)
        tm.add(host(S_m[lo:hi]), S_h)
        rs.rollback(S_h, None, x_h, M, acc[lo:hi])
        tr.add(host(S[lo:hi]), S_h)
        return to, tm, tr

    to, tm, tr = merge(over_unit_chunks(check, N, 16))
    say(f"  o: {to}; S after step_m: {tm}; S after rollback / commit: {tr}")
    assert to.n == M * N * vh * vd and tr.n == N * vh * kd * vd
    assert to.bad == 0 and tm.bad == 0 and tr.bad == 0


@pytest.mark.timeout(900)
def test_full_size_frontend_step_every_row(orc):
    """Workload 3 (front end + step, 128 sequences x 1 layer, 32 steps): every
    row's front-end outputs and every unit's o at every step against the
    oracle's own chain (front end, then step on the oracle's outputs); the
    conv history bit for bit and S after the last step."""
    cfg = synth.WORKLOADS[3]
    dims = cfg["dims"]
    vh, kh, kd, vd = dims
    B, T = cfg["seqs"], cfg["steps"]
    say(f"full size, every row: {cfg['name']}")
    gen = synth.make_gen(cfg["seed"], "cuda")
    S = synth.state(gen, B, dims, device="cuda")
    w = synth.frontend_weights(gen, dims, device="cuda")
    fe = synth.frontend_inputs(gen, B, dims, T=T, device="cuda")
    hist = fe["hist"]
    S0, hist0 = S.clone(), hist.clone()
    F = dict(q=torch.empty((T, B, kh, kd), device="cuda"),
             k=torch.empty((T, B, kh, kd), device="cuda"),
             v=torch.empty((T, B, vh, vd), device="cuda"),
             g=torch.empty((T, B, vh), device="cuda"),
             beta=torch.empty((T, B, vh), device="cuda"))
    O = torch.empty((T, B, vh, vd), device="cuda")
    for t in range(T):
        out = {n: F[n][t] for n in NAMES}
        gdn.frontend(fe["x"][t], w["Wa"], w["Wb"], w["A_log"], w["dt_bias"], fe["xc_raw"][t],
                     hist, w["conv_w"], dims, out=out)
        gdn.step(S, *(out[n] for n in NAMES), o=O[t])
    torch.cuda.synchronize()
    wh = {n: host(t) for n, t in w.items()}

    def check(lo, hi):
        tf, to, ts = Tally(), Tally(), Tally()
        n = hi - lo
        S_h, h_h = host(S0[lo:hi]), host(hist0[lo:hi])
        x_h, xc_h = host(fe["x"][:, lo:hi]), host(fe["xc_raw"][:, lo:hi])
        F_h = {k: host(F[k][:, lo:hi]) for k in NAMES}
        O_h = host(O[:, lo:hi])
        for t in range(T):
            ref = dict(q=np.zeros((n, kh, kd), np.float32), k=np.zeros((n, kh, kd), np.float32),
                       v=np.zeros((n, vh, vd), np.float32), g=np.zeros((n, vh), np.float32),
                       beta=np.zeros((n, vh), np.float32))
            orc.gdn_frontend(np.ascontiguousarray(x_h[t]), wh["Wa"], wh["Wb"], wh["A_log"],
                             wh["dt_bias"], np.ascontiguousarray(xc_h[t]), h_h, wh["conv_w"],
                             ref["q"], ref["k"], ref["v"], ref["g"], ref["beta"], dims)
            for k in NAMES:
                tf.add(F_h[k][t], ref[k])
            o_ref = np.zeros((n, vh, vd), np.float32)
            orc.gdn_step(S_h, *(ref[k] for k in NAMES), o_ref, dims)
            to.add(O_h[t], o_ref)
        ts.add(host(S[lo:hi]), S_h)
        hist_ok = host(hist[lo:hi]).tobytes() == h_h.tobytes()
        return tf, to, ts, hist_ok

    res = over_unit_chunks(check, B, 8)
    assert all(r[3] for r in res), "conv history differs from the oracle's"
    tf, to, ts = merge([r[:3] for r in res])
    say(f"  front end: {tf}; o: {to}; S: {ts}")
    assert to.n == T * B * vh * vd
    assert tf.bad == 0 and to.bad == 0 and ts.bad == 0
